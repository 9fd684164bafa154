"""GPU parity of the frame-valid masked squared-error loss with the fp64 oracle.

Tolerances (GPU vs oracle/loss.py):
  n_valid exact; loss and sum of squared errors within 1e-5 relative (fp32
  sums of bf16-exact or fp32 inputs); gradient per element within 1e-6
  relative (fp32 output) or 2^-8 relative (bf16 output, one rounding);
  padding rows of the gradient exactly zero.  The fused entry point and the
  split forward + backward give the same bits, and repeated calls too.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import loss as oloss
from oracle import seqids as osid
from tests._helpers import host64, ids_dev, to_dev

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-5
GRAD_RTOL = {"f32": 1e-6, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return pa_mod


def _run(pa, pred, target, ids, dtype, upstream):
    P, T, I = to_dev(pred, dtype), to_dev(target, dtype), ids_dev(ids)
    st = pa.masked_mse_fwd(P, T, I)
    g = pa.masked_mse_bwd(P, T, I, st, upstream)
    st2, g2 = pa.masked_mse_fwd_bwd(P, T, I, upstream)
    st3, g3 = pa.masked_mse_fwd_bwd(P, T, I, upstream)
    torch.cuda.synchronize()
    assert torch.equal(st, st2) and torch.equal(st2, st3), "fused / split / repeated stats differ"
    assert torch.equal(g.view(torch.int16) if dtype == "bf16" else g.view(torch.int32),
                       g2.view(torch.int16) if dtype == "bf16" else g2.view(torch.int32)), \
        "fused and split gradients differ"
    assert torch.equal(g2, g3)
    return st.cpu().numpy().astype(np.float64), host64(g)


def _check(pa, pred, target, ids, dtype, upstream=1.0):
    print(f"loss case n={len(ids)} C={pred.shape[1]} {dtype} upstream={upstream}", flush=True)
    st, g = _run(pa, pred, target, ids, dtype, upstream)
    loss, nv, dref = oloss.masked_mse(pred, target, ids, upstream)
    c = pred.shape[1]
    assert st[2] == nv
    assert abs(st[0] - loss) <= LOSS_RTOL * abs(loss), (st[0], loss)
    assert abs(st[1] - loss * nv * c) <= LOSS_RTOL * abs(loss * nv * c)
    if nv:
        assert abs(st[3] - 2.0 / (nv * c)) <= 1e-7 * 2.0 / (nv * c)
    else:
        assert st[0] == 0 and st[3] == 0
    keep = np.asarray(ids) >= 0
    assert np.isfinite(g).all()
    assert (g[~keep] == 0).all(), "padding rows of the gradient are not exactly zero"
    err = np.abs(g - dref)
    bound = GRAD_RTOL[dtype] * np.abs(dref) + 1e-30
    assert (err <= bound).all(), f"grad: max rel {float((err / (np.abs(dref) + 1e-30)).max()):.3e}"
    return st


def _frames_ids(vf, fp, tpf):
    return osid.seq_ids_from_valid_frames(np.array(vf, np.int32), fp, tpf)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_ragged(pa, dtype):
    ids = _frames_ids((3, 5, 0, 2), 6, 4)              # 96 rows, 56 padding
    p, t = wl.make_loss_values(len(ids), 24, dtype, seed=11)
    _check(pa, p, t, ids, dtype, upstream=1.7)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows_across_blocks_with_a_tail(pa, dtype):
    ids = _frames_ids((1000, 377, 1250, 3), 1251, 80)   # 400,320 rows, several per block
    p, t = wl.make_loss_values(len(ids), 16, dtype, seed=12)
    _check(pa, p, t, ids, dtype)


def test_padding_content_is_inert(pa):
    ids = _frames_ids((7, 2, 9), 9, 8)
    p, t = wl.make_loss_values(len(ids), 32, "bf16", seed=13)
    keep = ids >= 0
    p_bad = p.copy()
    p_bad[~keep] = wl.round_to_bf16(np.full_like(p[~keep], 3.0e38))  # huge, finite
    a, ga = _run(pa, p, t, ids, "bf16", 1.0)
    b, gb = _run(pa, p_bad, t, ids, "bf16", 1.0)
    assert np.array_equal(a, b) and np.array_equal(ga, gb)


def test_all_padding_and_single_row(pa):
    ids = np.full(50, -1, np.int32)
    p, t = wl.make_loss_values(50, 8, "f32", seed=14)
    st = _check(pa, p, t, ids, "f32")
    assert st[0] == 0 and st[2] == 0
    ids1 = np.zeros(1, np.int32)
    p1, t1 = wl.make_loss_values(1, 8, "f32", seed=15)
    _check(pa, p1, t1, ids1, "f32", upstream=-0.5)


def test_empty_input(pa):
    P = torch.empty((0, 16), dtype=torch.bfloat16, device="cuda")
    I = torch.empty(0, dtype=torch.int32, device="cuda")
    st, g = pa.masked_mse_fwd_bwd(P, P.clone(), I)
    st1 = pa.masked_mse_fwd(P, P.clone(), I)
    torch.cuda.synchronize()
    assert st.tolist() == [0.0, 0.0, 0.0, 0.0] and st1.tolist() == [0.0, 0.0, 0.0, 0.0]
    assert g.numel() == 0


@pytest.mark.parametrize("which,channels,dtype", [
    ("latent", 192, "bf16"),   # 4x288-frame pack, 32 video tokens per frame
    ("action", 32, "bf16"),    # same pack, 6 action tokens per frame
    ("long", 64, "f32"),       # 64,000-token mixed sequence (segment ids given)
])
def test_full_size_packs(pa, which, channels, dtype):
    s = wl.config(3) if which != "long" else wl.config(5)
    if which == "long":
        ids = s.segment_ids
    else:
        ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded,
                                             32 if which == "latent" else 6)
    p, t = wl.make_loss_values(len(ids), channels, dtype, seed=[16, channels])
    _check(pa, p, t, ids, dtype)
