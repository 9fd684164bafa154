"""Pins of the AdaLN oracle (oracle/adaln.py) against things other than itself.

  * torch's fp64 layer_norm (no affine) followed by the modulation, and torch
    autograd through it for dx, d_scale and d_shift;
  * central finite differences of sum(y * dy);
  * closed forms: a constant row normalises to 0, so y = shift; with zero
    modulation every valid row has mean 0 and variance var/(var + eps);
    with eps = 0, LayerNorm(a x + b) = LayerNorm(x) for a > 0;
  * padding rows and rows outside every segment give zeros and add nothing to
    the modulation gradients.
"""
import numpy as np
import pytest
import torch

from oracle import adaln as oada


def _case(seed=0, n=40, d=24, offsets=(0, 9, 9, 25, 36), pad=(3, 4, 20, 30, 31)):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)) * rng.uniform(0.5, 2.0, (n, 1)) + rng.standard_normal((n, 1))
    n_seg = len(offsets) - 1
    shift = 0.5 * rng.standard_normal((n_seg, d))
    scale = 0.5 * rng.standard_normal((n_seg, d))
    dy = rng.standard_normal((n, d))
    ids = np.zeros(n, np.int32)
    ids[list(pad)] = -1
    return x, dy, ids, np.array(offsets), shift, scale


def _torch_reference(x, dy, ids, offsets, shift, scale, eps):
    seg = oada.segment_of_rows(offsets, len(x))
    valid = (seg >= 0) & (np.asarray(ids) >= 0)
    X = torch.from_numpy(x).requires_grad_(True)
    SH = torch.from_numpy(shift).requires_grad_(True)
    SC = torch.from_numpy(scale).requires_grad_(True)
    idx = torch.from_numpy(np.where(valid, seg, 0))
    xhat = torch.nn.functional.layer_norm(X, (x.shape[1],), eps=eps)
    y = xhat * (1 + SC[idx]) + SH[idx]
    y = y * torch.from_numpy(valid.astype(np.float64))[:, None]
    (y * torch.from_numpy(dy)).sum().backward()
    return y.detach().numpy(), X.grad.numpy(), SH.grad.numpy(), SC.grad.numpy(), valid


@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_matches_torch_layer_norm_and_autograd(eps):
    x, dy, ids, off, shift, scale = _case()
    y, mean, rstd = oada.forward(x, ids, off, shift, scale, eps)
    dx, dsh, dsc = oada.backward(x, dy, ids, off, scale, eps)
    ty, tdx, tdsh, tdsc, valid = _torch_reference(x, dy, ids, off, shift, scale, eps)
    np.testing.assert_allclose(y, ty, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, tdx, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dsh, tdsh, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dsc, tdsc, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(mean[valid], x[valid].mean(axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(rstd[valid], 1 / np.sqrt(x[valid].var(axis=1) + eps), rtol=1e-12)
    assert (mean[~valid] == 0).all() and (rstd[~valid] == 0).all()


def test_finite_differences():
    x, dy, ids, off, shift, scale = _case(seed=2, n=12, d=8, offsets=(0, 5, 12), pad=(4, 9))
    dx, dsh, dsc = oada.backward(x, dy, ids, off, scale)
    f = lambda xx, sh, sc: float((oada.forward(xx, ids, off, sh, sc)[0] * dy).sum())  # noqa: E731
    h = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(20):
        i, j = int(rng.integers(12)), int(rng.integers(8))
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        assert abs((f(xp, shift, scale) - f(xm, shift, scale)) / (2 * h) - dx[i, j]) < 1e-6
    for s in range(2):
        for j in range(8):
            for tab, grad, which in ((shift, dsh, 0), (scale, dsc, 1)):
                tp, tm = tab.copy(), tab.copy()
                tp[s, j] += h
                tm[s, j] -= h
                args_p = (x, tp, scale) if which == 0 else (x, shift, tp)
                args_m = (x, tm, scale) if which == 0 else (x, shift, tm)
                assert abs((f(*args_p) - f(*args_m)) / (2 * h) - grad[s, j]) < 1e-6


def test_closed_forms():
    x, dy, ids, off, shift, scale = _case(seed=3)
    x[5] = 2.5                                     # constant row -> xhat = 0
    y, _, _ = oada.forward(x, ids, off, shift, scale)
    s = oada.segment_of_rows(off, len(x))[5]
    np.testing.assert_allclose(y[5], shift[s], rtol=0, atol=1e-12)
    eps = 1e-3
    y0, _, _ = oada.forward(x, ids, off, 0 * shift, 0 * scale, eps)
    seg = oada.segment_of_rows(off, len(x))
    valid = (seg >= 0) & (ids >= 0)
    valid[5] = False
    var = x[valid].var(axis=1)
    np.testing.assert_allclose(y0[valid].mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(y0[valid].var(axis=1), var / (var + eps), rtol=1e-12)
    xn = _case(seed=3)[0]                          # no constant row: eps = 0 is safe
    ya, _, _ = oada.forward(3.0 * xn - 7.0, ids, off, shift, scale, eps=0.0)
    yb, _, _ = oada.forward(xn, ids, off, shift, scale, eps=0.0)
    np.testing.assert_allclose(ya, yb, rtol=1e-10, atol=1e-11)


def test_padding_and_rows_outside_segments():
    x, dy, ids, off, shift, scale = _case(seed=4, offsets=(0, 9, 9, 25, 36))   # rows 36..39 outside
    y, mean, rstd = oada.forward(x, ids, off, shift, scale)
    dx, dsh, dsc = oada.backward(x, dy, ids, off, scale)
    dead = (ids < 0) | (np.arange(len(x)) >= 36)
    assert (y[dead] == 0).all() and (dx[dead] == 0).all()
    x2, dy2 = x.copy(), dy.copy()
    x2[dead] = 1e6
    dy2[dead] = -1e6
    dx2, dsh2, dsc2 = oada.backward(x2, dy2, ids, off, scale)
    assert np.array_equal(dsh, dsh2) and np.array_equal(dsc, dsc2)
    assert (dsh[1] == 0).all() and (dsc[1] == 0).all()      # empty segment 1


def test_offsets_are_clamped_and_made_monotone():
    seg = oada.segment_of_rows([-4, 3, 2, 7, 20], 10)      # -> 0, 3, 3, 7, 10
    assert seg.tolist() == [0, 0, 0, 2, 2, 2, 2, 3, 3, 3]
    assert oada.segment_of_rows([5, 5], 8).tolist() == [-1] * 8
