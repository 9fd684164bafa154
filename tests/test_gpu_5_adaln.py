"""GPU parity of the fused AdaLN forward / backward with the fp64 oracle.

Tolerances (GPU vs oracle/adaln.py, stated per output):
  fp32 inputs: y, dx: max|d| <= 1e-5 * max|ref|; mean, rstd: 1e-5 relative;
  bf16 inputs: y, dx per element |d| <= 2^-8 |ref| + 1e-4 * max|ref| (one bf16
               rounding of an fp32 result); mean, rstd: 1e-5 relative;
  d_shift, d_scale (fp32 sums over up to ~10^4 rows): max|d| <= 1e-4 * max|ref|.
Invalid rows (padding, outside every segment) must be exact zeros in y, dx,
mean and rstd; repeated calls must give the same bits.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import adaln as oada
from oracle import seqids as osid
from tests._helpers import host64, ids_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return pa_mod


def _run(pa, x, dy, ids, offsets, shift, scale, dtype, eps):
    X, DY = to_dev(x, dtype), to_dev(dy, dtype)
    I, OFF = ids_dev(ids), ids_dev(offsets)
    SH = torch.from_numpy(shift).cuda()
    SC = torch.from_numpy(scale).cuda()
    y, mean, rstd = pa.adaln_fwd(X, I, OFF, SH, SC, eps)
    dx, dsh, dsc = pa.adaln_bwd(X, DY, I, OFF, SC, mean, rstd)
    y2, mean2, rstd2 = pa.adaln_fwd(X, I, OFF, SH, SC, eps)
    dx2, dsh2, dsc2 = pa.adaln_bwd(X, DY, I, OFF, SC, mean2, rstd2)
    torch.cuda.synchronize()
    for a, b in ((y, y2), (mean, mean2), (rstd, rstd2), (dx, dx2), (dsh, dsh2), (dsc, dsc2)):
        assert torch.equal(a, b), "repeated calls differ"
    return [host64(t) for t in (y, mean, rstd, dx, dsh, dsc)]


def _close_elem(name, got, ref, dtype):
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 1e-5 * scale, f"{name}: max rel {err.max() / scale:.3e}"
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * scale
        bad = err > bound
        assert not bad.any(), f"{name}: {int(bad.sum())} elements out of tolerance, " \
                              f"worst {float((err - bound).max()):.3e}"


def _check(pa, x, dy, ids, offsets, shift, scale, dtype, eps=1e-6):
    n, d = x.shape
    print(f"adaln case n={n} D={d} S={len(offsets) - 1} {dtype}", flush=True)
    y, mean, rstd, dx, dsh, dsc = _run(pa, x, dy, ids, offsets, shift, scale, dtype, eps)
    ry, rmean, rrstd = oada.forward(x, ids, offsets, shift, scale, eps)
    rdx, rdsh, rdsc = oada.backward(x, dy, ids, offsets, scale, eps)
    seg = oada.segment_of_rows(offsets, n)
    valid = (seg >= 0) & (np.asarray(ids) >= 0)
    for name, g in (("y", y), ("dx", dx)):
        assert np.isfinite(g).all() and (g[~valid] == 0).all(), f"{name}: invalid rows not zero"
    assert (mean[~valid] == 0).all() and (rstd[~valid] == 0).all()
    if valid.any():
        _close_elem("y", y[valid], ry[valid], dtype)
        _close_elem("dx", dx[valid], rdx[valid], dtype)
        np.testing.assert_allclose(mean[valid], rmean[valid], rtol=1e-5,
                                   atol=1e-5 * np.abs(rmean[valid]).max())
        np.testing.assert_allclose(rstd[valid], rrstd[valid], rtol=1e-5)
    for name, g, r in (("d_shift", dsh, rdsh), ("d_scale", dsc, rdsc)):
        assert g.shape == r.shape
        if r.size == 0:
            continue
        sc = max(float(np.abs(r).max()), 1e-30)
        assert np.abs(g - r).max() <= 1e-4 * sc, f"{name}: max rel {np.abs(g - r).max() / sc:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [72, 520, 3072])
def test_small_ragged_segments(pa, dtype, d):
    n = 300
    offsets = np.array([5, 100, 100, 250], np.int32)      # rows 0-4 and 250-299 in no segment
    ids = np.zeros(n, np.int32)
    ids[[7, 50, 51, 99, 100, 180]] = -1
    x, dy, shift, scale = wl.make_adaln_values(n, d, 3, dtype, seed=[21, d])
    _check(pa, x, dy, ids, offsets, shift, scale, dtype)


def test_widest_rows_and_odd_offsets(pa):
    n, d = 200, 4096
    offsets = np.array([-7, 30, 20, 150, 999], np.int32)   # clamped to 0, 30, 30, 150, 200
    ids = np.where(np.arange(n) % 17 == 3, -1, 0).astype(np.int32)
    x, dy, shift, scale = wl.make_adaln_values(n, d, 4, "bf16", seed=22)
    _check(pa, x, dy, ids, offsets, shift, scale, "bf16", eps=1e-5)


def test_no_segments_and_empty(pa):
    x, dy, shift, scale = wl.make_adaln_values(40, 64, 0, "bf16", seed=23)
    _check(pa, x, dy, np.zeros(40, np.int32), np.array([0], np.int32), shift, scale, "bf16")
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    I = torch.empty(0, dtype=torch.int32, device="cuda")
    OFF = torch.zeros(3, dtype=torch.int32, device="cuda")
    SH = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    y, mean, rstd = pa.adaln_fwd(X, I, OFF, SH, SH.clone())
    dx, dsh, dsc = pa.adaln_bwd(X, X.clone(), I, OFF, SH, mean, rstd)
    torch.cuda.synchronize()
    assert y.numel() == 0 and (dsh == 0).all() and (dsc == 0).all()


def test_frame_padded_pack_full_size(pa):
    """The 4 x 288-frame pack: 36,864 rows of 3072 features, one segment per episode."""
    s = wl.config(3)
    ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    per = s.frames_padded * s.q_tokens_per_frame
    offsets = (np.arange(s.n_episodes + 1) * per).astype(np.int32)
    x, dy, shift, scale = wl.make_adaln_values(s.nq, 3072, s.n_episodes, "bf16", seed=24)
    _check(pa, x, dy, ids, offsets, shift, scale, "bf16")


def test_unpadded_pack_full_size(pa):
    """The first 68,000-token unpadded pack of the episode stream, 3072 features."""
    import packed_variable_length_amd as pam
    lengths = wl.episode_stream()
    pack_of, _ = pam.plan_token_packs(lengths, wl.UNPADDED_BUDGET)
    sel = lengths[pack_of == 0]
    n = wl.UNPADDED_BUDGET
    ids = osid.seq_ids_from_lengths(sel, n)
    offsets = np.concatenate([[0], np.cumsum(sel)]).astype(np.int32)
    x, dy, shift, scale = wl.make_adaln_values(n, 3072, len(sel), "bf16", seed=25)
    _check(pa, x, dy, ids, offsets, shift, scale, "bf16")
