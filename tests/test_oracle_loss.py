"""Pins of the masked-loss oracle (oracle/loss.py) against things other than itself.

The loss follows the "LingBot-VA packing" report, section 2.1 (compute_loss:
padding frames excluded from the latent/action loss means).  Pins:
  * torch's mean-squared-error routine over only the valid rows, and torch
    autograd through it for the gradient (a library routine, not the loop);
  * the per-frame reading of the pages: the mean over valid frames of each
    frame's mean squared error (equal tokens per frame);
  * packed equals pooled: the loss of a padded pack equals the loss of the
    valid rows concatenated without padding, whatever the padding holds
    (the report's check that a packed batch and separate episodes agree);
  * closed forms (constant offset a gives a^2; all padding gives 0);
  * central finite differences of the loss for the gradient.
"""
import numpy as np
import pytest
import torch

from oracle import loss as oloss
from oracle import seqids as osid


def _case(seed=0, vf=(3, 5, 0, 2), fp=6, tpf=4, c=16):
    rng = np.random.default_rng(seed)
    ids = osid.seq_ids_from_valid_frames(np.array(vf, np.int32), fp, tpf)
    n = len(ids)
    return rng.standard_normal((n, c)), rng.standard_normal((n, c)), ids


def test_matches_torch_mse_on_valid_rows_and_autograd():
    p, t, ids = _case()
    loss, nv, dp = oloss.masked_mse(p, t, ids, upstream=1.7)
    keep = torch.from_numpy(np.asarray(ids) >= 0)
    P = torch.from_numpy(p).requires_grad_(True)
    ref = torch.nn.functional.mse_loss(P[keep], torch.from_numpy(t)[keep])
    (1.7 * ref).backward()
    assert nv == int(keep.sum())
    assert abs(loss - ref.item()) <= 1e-14 * max(1.0, abs(ref.item()))
    np.testing.assert_allclose(dp, P.grad.numpy(), rtol=1e-13, atol=1e-16)


def test_equals_mean_over_valid_frames_of_frame_means():
    vf, fp, tpf, c = (3, 5, 0, 2), 6, 4, 16
    p, t, ids = _case(vf=vf, fp=fp, tpf=tpf, c=c)
    per_frame = ((p - t) ** 2).reshape(len(vf), fp, tpf * c).mean(axis=2)   # [B, F]
    frame_valid = np.arange(fp)[None, :] < np.array(vf)[:, None]
    ref = per_frame[frame_valid].mean()
    loss, _, _ = oloss.masked_mse(p, t, ids)
    assert abs(loss - ref) <= 1e-14 * ref


def test_packed_equals_pooled_and_padding_is_inert():
    p, t, ids = _case(seed=3)
    keep = np.asarray(ids) >= 0
    pooled, nv, dpool = oloss.masked_mse(p[keep], t[keep], np.zeros(int(keep.sum()), np.int32))
    packed, nv2, dpack = oloss.masked_mse(p, t, ids)
    assert nv == nv2 and abs(pooled - packed) <= 1e-15 * pooled
    np.testing.assert_array_equal(dpack[keep], dpool)
    p2 = p.copy()
    p2[~keep] = 1e6                      # garbage predictions on padding frames
    packed2, _, dpack2 = oloss.masked_mse(p2, t, ids)
    assert packed2 == packed
    assert (dpack2[~keep] == 0).all() and (dpack[~keep] == 0).all()


@pytest.mark.parametrize("a", [0.0, 0.5, -3.0])
def test_constant_offset_closed_form(a):
    _, t, ids = _case(seed=5)
    loss, _, dp = oloss.masked_mse(t + a, t, ids)
    assert abs(loss - a * a) <= 1e-14 * max(1.0, a * a)
    keep = np.asarray(ids) >= 0
    nv, c = int(keep.sum()), t.shape[1]
    np.testing.assert_allclose(dp[keep], 2 * a / (nv * c), rtol=1e-14, atol=0)


def test_all_padding_gives_zero():
    p, t, ids = _case(vf=(0, 0), fp=4, tpf=2, c=8)
    loss, nv, dp = oloss.masked_mse(p, t, ids)
    assert loss == 0.0 and nv == 0 and (dp == 0).all()


def test_gradient_by_finite_differences():
    p, t, ids = _case(seed=7, vf=(2, 1), fp=3, tpf=2, c=8)
    _, _, dp = oloss.masked_mse(p, t, ids)
    h = 1e-6
    rng = np.random.default_rng(1)
    for _ in range(12):
        i, j = int(rng.integers(p.shape[0])), int(rng.integers(p.shape[1]))
        pp, pm = p.copy(), p.copy()
        pp[i, j] += h
        pm[i, j] -= h
        fd = (oloss.masked_mse(pp, t, ids)[0] - oloss.masked_mse(pm, t, ids)[0]) / (2 * h)
        assert abs(fd - dp[i, j]) <= 1e-7, (i, j, fd, dp[i, j])
