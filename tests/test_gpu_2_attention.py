"""GPU parity of packed masked attention (forward and backward) with the fp64 oracle.

Small packs are compared element by element on every head (the full-size
workloads are in test_gpu_6_full_parity.py).
Tolerances: see tests/_helpers.py.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oatt
from oracle import seqids as osid
from tests._helpers import (Guarded, compare, compare_lse, host64, ids_dev, row_has_pair,
                            to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return pa_mod


def _ids_from_spec(pa, s):
    """(oracle ids, GPU ids) built independently for each side."""
    if s.segment_ids is not None:
        return (s.segment_ids, s.segment_ids), (ids_dev(s.segment_ids), ids_dev(s.segment_ids))
    qo = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    ko = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.kv_tokens_per_frame)
    vf = ids_dev(s.valid_frames)
    qg = pa.seq_ids_from_valid_frames(vf, s.frames_padded, s.q_tokens_per_frame)
    kg = pa.seq_ids_from_valid_frames(vf, s.frames_padded, s.kv_tokens_per_frame)
    return (qo, ko), (qg, kg)


def _run_gpu(pa, q, k, v, do, qg, kg, dtype, scale, bq=128, bkv=128):
    """Forward and backward with every output, the mask storage and the
    workspace inside guard bands (interiors pre-filled with a NaN canary)."""
    Q, K, V, DO = (to_dev(a, dtype) for a in (q, k, v, do))
    nq, nkv, H, d = Q.shape[0], K.shape[0], Q.shape[1], Q.shape[2]
    mstore = Guarded((pa.build_block_mask_bytes(nq, nkv, bq, bkv),), torch.uint8)
    mask = pa.build_block_mask(qg, kg, bq, bkv, storage=mstore.tensor)
    go, glse = Guarded(Q.shape, Q.dtype), Guarded((H, nq), torch.float32)
    o, lse = pa.attn_packed_fwd(Q, K, V, qg, kg, mask, scale, out=go.tensor, lse=glse.tensor)
    gq, gk, gv = Guarded(Q.shape, Q.dtype), Guarded(K.shape, K.dtype), Guarded(V.shape, V.dtype)
    ws = Guarded((pa.attn_packed_bwd_workspace_bytes(Q.dtype, nq, nkv, H, d),), torch.uint8)
    dq, dk, dv = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask, scale,
                                    workspace=ws.tensor, grads=(gq.tensor, gk.tensor, gv.tensor))
    torch.cuda.synchronize()
    for name, g in (("mask storage", mstore), ("o", go), ("lse", glse), ("dq", gq), ("dk", gk),
                    ("dv", gv), ("workspace", ws)):
        g.check(name)
    return dict(o=host64(o), lse=lse.cpu().numpy().astype(np.float64), dq=host64(dq),
                dk=host64(dk), dv=host64(dv))


def _check(got, ref, qo, ko, dtype, heads=None):
    q_ok, k_ok = row_has_pair(qo, ko)
    out = {}
    out["o"] = compare("O", got["o"], ref["o"], q_ok, dtype, heads)
    out["dq"] = compare("dQ", got["dq"], ref["dq"], q_ok, dtype, heads)
    out["dk"] = compare("dK", got["dk"], ref["dk"], k_ok, dtype, heads)
    out["dv"] = compare("dV", got["dv"], ref["dv"], k_ok, dtype, heads)
    compare_lse(got["lse"], ref["lse"], heads)
    return out


def _spec(valid, fp, tq, tk, heads, d, dtype, seed):
    return wl.PackSpec(f"case-{seed}", heads=heads, head_dim=d, dtype=dtype, seed=seed,
                       value_std=0.5 if dtype == "bf16" else 1.0,
                       valid_frames=np.array(valid, np.int32), frames_padded=fp,
                       q_tokens_per_frame=tq, kv_tokens_per_frame=tk)


SMALL = [
    # valid frames, padded frames, q tok/frame, kv tok/frame, heads, head_dim
    ([5, 9, 0, 3, 7], 9, 32, 32, 2, 128),   # 1440 tokens: 12 tiles, ragged tail, empty episode
    ([5, 9, 3], 9, 6, 32, 2, 128),          # cross-attention, nq != nkv
    ([4, 1, 6], 6, 32, 32, 3, 64),          # head_dim 64
    ([17, 2], 20, 16, 16, 1, 128),          # partial tiles in the middle of the pack
    ([3, 5, 2], 8, 4, 4, 1, 64),            # the tiny pack in bf16
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_bf16_small_packs_all_heads(pa, case):
    valid, fp, tq, tk, H, d = SMALL[case]
    s = _spec(valid, fp, tq, tk, H, d, "bf16", 10 + case)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    got = _run_gpu(pa, q, k, v, do, qg, kg, "bf16", s.scale)
    ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    _check(got, ref, qo, ko, "bf16")


# head counts that are multiples of 8 take the XCD head walk of the grid
# mapping (XCD x runs heads x, x + 8, ...), the branch every production shape
# (24 heads) takes: every head is compared, with NaN-filled outputs
XCD_HEADS = [
    ([5, 9, 0, 3, 7], 9, 32, 32, 8, 128),   # 1440 tokens, self
    ([5, 9, 3], 9, 6, 32, 8, 128),          # cross-attention
    ([5, 9, 0, 3, 7], 9, 32, 32, 16, 64),   # 64-wide heads
    ([9, 2, 6], 9, 32, 32, 16, 128),        # 16 heads: two heads per XCD
    ([4, 7], 8, 12, 32, 24, 64),            # 24 heads, cross, 64-wide
]


@pytest.mark.parametrize("case", range(len(XCD_HEADS)))
def test_bf16_xcd_head_walk_all_heads(pa, case):
    valid, fp, tq, tk, H, d = XCD_HEADS[case]
    s = _spec(valid, fp, tq, tk, H, d, "bf16", 60 + case)
    print(f"[xcd heads] H={H} d={d} nq={s.nq} nkv={s.nkv}", flush=True)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    got = _run_gpu(pa, q, k, v, do, qg, kg, "bf16", s.scale)
    ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    _check(got, ref, qo, ko, "bf16")
    for h in range(H):  # each head on its own: a swapped or missing head fails here
        _check(got, ref, qo, ko, "bf16", heads=[h])


@pytest.mark.parametrize("seed", range(3))
def test_bf16_interleaved_ids(pa, seed):
    rng = np.random.default_rng(seed)
    nq, nkv, H, d = 700, 650 if seed else 700, 2, 128
    qo = rng.integers(-1, 5, nq).astype(np.int32)
    ko = qo.copy() if seed == 0 else rng.integers(-1, 4, nkv).astype(np.int32)  # id 4: no keys
    s = wl.PackSpec("interleaved", heads=H, head_dim=d, dtype="bf16", seed=seed, value_std=0.5,
                    segment_ids=qo)
    q, _, _, do = wl.make_values(s)
    kk = wl.round_to_bf16(rng.standard_normal((nkv, H, d)).astype(np.float32) * 0.5)
    vv = wl.round_to_bf16(rng.standard_normal((nkv, H, d)).astype(np.float32) * 0.5)
    got = _run_gpu(pa, q, kk, vv, do, ids_dev(qo), ids_dev(ko), "bf16", s.scale)
    ref = oatt.forward_backward(q, kk, vv, do, qo, ko, s.scale)
    _check(got, ref, qo, ko, "bf16")


def _segments(lengths, gaps):
    """Ids for consecutive segments 0, 1, ... of the given lengths, each preceded
    by a run of `gaps[i]` padding tokens (-1)."""
    parts = []
    for i, (n, g) in enumerate(zip(lengths, gaps)):
        parts += [np.full(g, -1, np.int32), np.full(n, i, np.int32)]
    return np.concatenate(parts)


# segment lengths around the 64-token sub-tile and 128-token tile sizes, with
# padding runs that shift each segment against the tile grid
BOUNDARY_LEN = [1, 63, 64, 65, 127, 128, 129, 191, 256, 257]
BOUNDARY_GAP = [0, 5, 0, 64, 1, 0, 127, 3, 0, 33]


@pytest.mark.parametrize("cross,d", [(False, 128), (True, 128), (False, 64), (True, 64)])
def test_bf16_boundary_lengths(pa, cross, d):
    rng = np.random.default_rng(31 + cross + d)
    qo = _segments(BOUNDARY_LEN, BOUNDARY_GAP)
    # cross: the same segments with other lengths on the key side (one empty)
    ko = (_segments([129, 64, 1, 0, 200, 63, 128, 65, 127, 300], [2, 0, 64, 7, 0, 1, 0, 0, 129, 5])
          if cross else qo.copy())
    H = 3 if d == 64 else 2
    s = wl.PackSpec("boundary", heads=H, head_dim=d, dtype="bf16", seed=31, value_std=0.5,
                    segment_ids=qo)
    q, _, _, do = wl.make_values(s)
    nkv = len(ko)
    kk = wl.round_to_bf16(rng.standard_normal((nkv, H, d)).astype(np.float32) * 0.5)
    vv = wl.round_to_bf16(rng.standard_normal((nkv, H, d)).astype(np.float32) * 0.5)
    got = _run_gpu(pa, q, kk, vv, do, ids_dev(qo), ids_dev(ko), "bf16", s.scale)
    ref = oatt.forward_backward(q, kk, vv, do, qo, ko, s.scale)
    _check(got, ref, qo, ko, "bf16")


def test_bf16_score_jump_late_in_the_walk(pa):
    """Keys deep in the walk whose scores exceed every earlier score of a row by
    far more than the fp32 range of exp2 (k = 60 q of that row, about 245 in
    log2 units), and a large negative score: O, LSE and dV still match the
    oracle, dQ and dK are finite.  The forward raises a row's running max only
    when a score passes it by more than its lazy threshold, and then rescales
    O and the row sum; a forward that missed that rescale would return inf or
    NaN here.  (dQ and dK of a row whose softmax is one-hot
    come from dP - Delta, a difference of two nearly equal terms of which
    Delta uses the bf16-rounded O, so their relative error there is that of
    bf16 rounding, not of the kernels.)"""
    n, H, d = 900, 2, 128
    ids = np.zeros(n, np.int32)
    ids[850:] = 1
    s = wl.PackSpec("jump", heads=H, head_dim=d, dtype="bf16", seed=77, value_std=0.5,
                    segment_ids=ids)
    q, k, v, do = wl.make_values(s)
    k = k.copy()
    for h in range(H):
        k[700, h] = wl.round_to_bf16(60.0 * q[5, h])        # query 5 (tile 0) meets key 700 (tile 5)
        k[300, h] = wl.round_to_bf16(40.0 * q[140 + h, h])  # queries of tile 1, key of tile 2
    k[640, 1] = wl.round_to_bf16(-30.0 * q[200, 1])
    got = _run_gpu(pa, q, k, v, do, ids_dev(ids), ids_dev(ids), "bf16", s.scale)
    ref = oatt.forward_backward(q, k, v, do, ids, ids, s.scale)
    assert ref["lse"][0, 5] > 100.0                          # the jump is real
    q_ok, k_ok = row_has_pair(ids, ids)
    compare("O", got["o"], ref["o"], q_ok, "bf16")
    compare("dV", got["dv"], ref["dv"], k_ok, "bf16")
    compare_lse(got["lse"], ref["lse"])
    assert np.isfinite(got["dq"]).all() and np.isfinite(got["dk"]).all()


def test_bf16_all_padding_pack(pa):
    s = _spec([0, 0], 4, 32, 32, 2, 128, "bf16", 3)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    got = _run_gpu(pa, q, k, v, do, qg, kg, "bf16", s.scale)
    for name in ("o", "dq", "dk", "dv"):
        assert (got[name] == 0).all()
    assert np.isneginf(got["lse"]).all()


def test_fp32_tiny_pack(pa):
    s = wl.config(1)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    for bq, bkv in ((32, 32), (64, 64), (128, 128), (32, 128)):
        got = _run_gpu(pa, q, k, v, do, qg, kg, "f32", s.scale, bq, bkv)
        ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
        _check(got, ref, qo, ko, "f32")


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_multi_tile_and_cross(pa, d):
    for spec in (_spec([5, 9, 0, 3], 9, 16, 16, 2, d, "f32", 7),
                 _spec([5, 9, 3], 9, 6, 32, 2, d, "f32", 8)):
        q, k, v, do = wl.make_values(spec)
        (qo, ko), (qg, kg) = _ids_from_spec(pa, spec)
        got = _run_gpu(pa, q, k, v, do, qg, kg, "f32", spec.scale, 64, 32)
        ref = oatt.forward_backward(q, k, v, do, qo, ko, spec.scale)
        _check(got, ref, qo, ko, "f32")


def test_no_leakage_across_episodes(pa):
    # 24 tokens per frame: query and key tiles straddle two episodes' valid tokens
    s = _spec([9, 7, 9, 8], 9, 24, 24, 2, 128, "bf16", 21)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    base = _run_gpu(pa, q, k, v, do, qg, kg, "bf16", s.scale)
    ep = qo == 1
    q2, k2, v2, do2 = (a.copy() for a in (q, k, v, do))
    for a in (q2, k2, v2, do2):
        a[ep] = wl.round_to_bf16(a[ep] * 1.5 + 0.25)
    pert = _run_gpu(pa, q2, k2, v2, do2, qg, kg, "bf16", s.scale)
    for name in ("o", "dq", "dk", "dv"):
        assert np.array_equal(pert[name][~ep], base[name][~ep]), name
        assert not np.array_equal(pert[name][ep], base[name][ep]), name
    assert np.array_equal(pert["lse"][:, ~ep], base["lse"][:, ~ep])


def test_backward_deterministic_and_mask_hazard(pa):
    s = _spec([5, 9, 3], 9, 32, 32, 2, 128, "bf16", 4)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    Q, K, V, DO = (to_dev(a, "bf16") for a in (q, k, v, do))
    mask = pa.build_block_mask(qg, kg)
    o, lse = pa.attn_packed_fwd(Q, K, V, qg, kg, mask)
    # a forward of another shape in between must not corrupt this backward
    other = ids_dev(np.zeros(300, np.int32))
    mask_other = pa.build_block_mask(other, other)
    X = to_dev(np.zeros((300, 2, 128), np.float32), "bf16")
    pa.attn_packed_fwd(X, X, X, other, other, mask_other)
    with pytest.raises(pa.PackAttnError) as ei:
        pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask_other)
    assert ei.value.status == -5
    g1 = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask)
    g2 = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    got = dict(o=host64(o), lse=lse.cpu().numpy().astype(np.float64), dq=host64(g1[0]),
               dk=host64(g1[1]), dv=host64(g1[2]))
    _check(got, ref, qo, ko, "bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_backward_stages_match_the_combined_call(pa, dtype, d):
    """The two stage entry points (row terms + dQ, then dK/dV) called one by one,
    into buffers of their own, give gradients bit-identical to attn_packed_bwd
    (the same kernels) and within tolerance of the oracle; the row terms the dQ
    stage writes agree with the preprocess entry point's, and dK/dV from the
    preprocess's row terms is within tolerance too."""
    s = _spec([5, 9, 3], 9, 32, 32, 2, d, dtype, 6)
    print(f"[stages] {dtype} d={d} nq={s.nq}", flush=True)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    Q, K, V, DO = (to_dev(a, dtype) for a in (q, k, v, do))
    mask = pa.build_block_mask(qg, kg)
    o, lse = pa.attn_packed_fwd(Q, K, V, qg, kg, mask, s.scale)
    whole = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask, s.scale)
    ws = torch.empty(pa.attn_packed_bwd_workspace_bytes(Q.dtype, s.nq, s.nkv, 2, d),
                     dtype=torch.uint8, device=Q.device)
    dq = pa.attn_packed_bwd_dq(Q, K, V, o, DO, lse, ws, qg, kg, mask, s.scale)
    dk, dv = pa.attn_packed_bwd_dkdv(Q, K, V, DO, lse, ws, qg, kg, mask, s.scale)
    for a, b in zip(whole, (dq, dk, dv)):
        assert torch.equal(a, b)
    # the row terms the dQ stage leaves in the workspace equal the preprocess's
    # up to summation order: Delta = rowsum(dO * O) and the LSE in log2 units
    rows = ws[:2 * 2 * s.nq * 4].view(torch.float32).view(2, 2, s.nq).clone()
    ws2 = pa.attn_packed_bwd_preprocess(o, DO, lse)
    pre = ws2[:2 * 2 * s.nq * 4].view(torch.float32).view(2, 2, s.nq)
    assert torch.equal(torch.isinf(rows[1]), torch.isinf(pre[1]))
    fin = torch.isfinite(pre[1])
    assert torch.allclose(rows[1][fin], pre[1][fin], rtol=0, atol=0)
    assert torch.allclose(rows[0], pre[0], rtol=1e-5, atol=1e-5)
    dk2, dv2 = pa.attn_packed_bwd_dkdv(Q, K, V, DO, lse, ws2, qg, kg, mask, s.scale)
    ref0 = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    q_ok, k_ok = row_has_pair(qo, ko)
    compare("dK (preprocess row terms)", host64(dk2), ref0["dk"], k_ok, dtype)
    compare("dV (preprocess row terms)", host64(dv2), ref0["dv"], k_ok, dtype)
    ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    got = dict(o=host64(o), lse=lse.cpu().numpy().astype(np.float64), dq=host64(dq),
               dk=host64(dk), dv=host64(dv))
    _check(got, ref, qo, ko, dtype)


def test_handover_wait_that_runs_out_poisons_dv(pa):
    """The dK/dV kernel (bf16, 128-wide heads) hands P from one wave to the
    other through LDS behind a bounded wait.  Forced from the host to run out
    (a bound of zero polls), the waiting waves write NaN into their dv rows
    instead of values -- every key tile with work has such a wait -- and the
    kernel still ends normally; back at the default bound the results match
    the oracle again.  The device-side count of such waves
    (pa_handover_failures) is nonzero after the forced run and zero after the
    normal one."""
    s = _spec([5, 9, 3], 9, 32, 32, 2, 128, "bf16", 4)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    Q, K, V, DO = (to_dev(a, "bf16") for a in (q, k, v, do))
    mask = pa.build_block_mask(qg, kg)
    o, lse = pa.attn_packed_fwd(Q, K, V, qg, kg, mask)
    ntiles = (s.nkv + 127) // 128
    tile_has_work = np.array([(ko[128 * t:128 * (t + 1)] >= 0).any() for t in range(ntiles)])
    rows_with_work = np.repeat(tile_has_work, 128)[: s.nkv]
    assert tile_has_work.any() and not tile_has_work.all()
    pa.pa_handover_failures(reset=True)
    default = pa.pa_test_set_handover_spin_limit(0)
    try:
        assert default == 1 << 20
        _, _, dv = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask)
        torch.cuda.synchronize()
        dv = host64(dv)
    finally:
        assert pa.pa_test_set_handover_spin_limit(-1) == 0
    assert np.isnan(dv[rows_with_work]).all()
    assert (dv[~rows_with_work] == 0).all()
    assert pa.pa_handover_failures(reset=True) > 0
    g = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask)
    torch.cuda.synchronize()
    assert pa.pa_handover_failures() == 0
    ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    got = dict(o=host64(o), lse=lse.cpu().numpy().astype(np.float64), dq=host64(g[0]),
               dk=host64(g[1]), dv=host64(g[2]))
    _check(got, ref, qo, ko, "bf16")


def test_binding_refuses_wrong_output_buffers(pa):
    """The C ABI takes bare pointers, so the binding must refuse an output or
    workspace of the wrong shape, dtype or layout before anything is launched."""
    s = _spec([5, 9, 3], 9, 6, 32, 2, 128, "bf16", 5)  # cross: nq != nkv
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids_from_spec(pa, s)
    Q, K, V, DO = (to_dev(a, "bf16") for a in (q, k, v, do))
    mask = pa.build_block_mask(qg, kg)
    nq, nkv, H, d = Q.shape[0], K.shape[0], Q.shape[1], Q.shape[2]
    dev = Q.device
    bad_o = [torch.empty((nq - 1, H, d), dtype=torch.bfloat16, device=dev),
             torch.empty((nq, H, d), dtype=torch.float32, device=dev),
             torch.empty((nq, H, 2 * d), dtype=torch.bfloat16, device=dev)[..., :d]]
    for o_bad in bad_o:
        with pytest.raises(ValueError):
            pa.attn_packed_fwd(Q, K, V, qg, kg, mask, out=o_bad)
    with pytest.raises(ValueError):
        pa.attn_packed_fwd(Q, K, V, qg, kg, mask,
                           lse=torch.empty((H, nq - 1), dtype=torch.float32, device=dev))
    o, lse = pa.attn_packed_fwd(Q, K, V, qg, kg, mask)
    good = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    for i, shape in ((0, (nq, H, d - 8)), (1, (nq, H, d)), (2, (nkv + 1, H, d))):
        grads = list(good)
        grads[i] = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        with pytest.raises(ValueError):
            pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask, grads=tuple(grads))
    with pytest.raises(ValueError):  # seq ids of the wrong length
        pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg[:-1].contiguous(), kg, mask)
    with pytest.raises(ValueError):
        pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask,
                           workspace=torch.empty(16, dtype=torch.float32, device=dev))
    ws = pa.attn_packed_bwd_preprocess(o, DO, lse)
    with pytest.raises(ValueError):
        pa.attn_packed_bwd_dq(Q, K, V, o, DO, lse, ws, qg, kg, mask, dq=torch.empty_like(K))
    with pytest.raises(ValueError):
        pa.attn_packed_bwd_dkdv(Q, K, V, DO, lse, ws, qg, kg, mask, dk=torch.empty_like(Q))
    with pytest.raises(ValueError):
        pa.attn_packed_bwd_dq(Q, K, V, o, DO, lse[:, :-1].contiguous(), ws, qg, kg, mask)
    with pytest.raises(ValueError):
        pa.attn_packed_bwd_dkdv(Q, K, V, DO, lse, ws, qg, kg[:-1].contiguous(), mask)
    # the checks refused everything above before a launch: the good call still matches
    torch.cuda.synchronize()
    dq, dk, dv = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask, s.scale, grads=good)
    ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    got = dict(o=host64(o), lse=lse.cpu().numpy().astype(np.float64), dq=host64(dq),
               dk=host64(dk), dv=host64(dv))
    _check(got, ref, qo, ko, "bf16")
