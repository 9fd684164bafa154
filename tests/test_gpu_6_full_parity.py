"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (128 x 128 mask tiles, 24 heads x 128, bf16).

Every head of every output is checked on the device: values finite, rows with
no allowed pair exactly zero, the LSE -inf pattern exactly that of the rows
without an allowed key.  Values are compared with the fp64 oracle head by head:
all 24 heads of the 4 x 288-frame and 4 x 120-frame packs, four heads of the
64k mixed pack and of the 4 x 288 pack scattered in 512-token pieces, and one head per batch of all 40 batches of the length-bucketed
sweep, self- and cross-attention (the head rotates over the batches, so every
head is compared somewhere).  Outputs sit inside guard bands.  Tolerances: see
tests/_helpers.py.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oatt
from oracle import seqids as osid
from tests._helpers import Guarded, compare, compare_lse, host64, ids_dev, row_has_pair

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return pa_mod


def _ids(pa, s):
    """(oracle ids, GPU ids), each side built on its own."""
    if s.segment_ids is not None:
        return (s.segment_ids, s.segment_ids), (ids_dev(s.segment_ids), ids_dev(s.segment_ids))
    qo = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    ko = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.kv_tokens_per_frame)
    vf = ids_dev(s.valid_frames)
    qg = pa.seq_ids_from_valid_frames(vf, s.frames_padded, s.q_tokens_per_frame)
    kg = pa.seq_ids_from_valid_frames(vf, s.frames_padded, s.kv_tokens_per_frame)
    assert np.array_equal(qg.cpu().numpy(), qo) and np.array_equal(kg.cpu().numpy(), ko)
    return (qo, ko), (qg, kg)


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()


def _run(pa, Q, K, V, DO, qg, kg, scale):
    nq, nkv, H, d = Q.shape[0], K.shape[0], Q.shape[1], Q.shape[2]
    mstore = Guarded((pa.build_block_mask_bytes(nq, nkv, 128, 128),), torch.uint8)
    mask = pa.build_block_mask(qg, kg, 128, 128, storage=mstore.tensor)
    go, glse = Guarded(Q.shape, Q.dtype), Guarded((H, nq), torch.float32)
    o, lse = pa.attn_packed_fwd(Q, K, V, qg, kg, mask, scale, out=go.tensor, lse=glse.tensor)
    gq, gk, gv = Guarded(Q.shape, Q.dtype), Guarded(K.shape, K.dtype), Guarded(V.shape, V.dtype)
    ws = Guarded((pa.attn_packed_bwd_workspace_bytes(Q.dtype, nq, nkv, H, d),), torch.uint8)
    pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask, scale, workspace=ws.tensor,
                       grads=(gq.tensor, gk.tensor, gv.tensor))
    torch.cuda.synchronize()
    for name, g in (("mask storage", mstore), ("o", go), ("lse", glse), ("dq", gq), ("dk", gk),
                    ("dv", gv), ("workspace", ws)):
        g.check(name)
    return dict(o=o, lse=lse, dq=gq.tensor, dk=gk.tensor, dv=gv.tensor)


def _device_checks(got, qo, ko):
    """All heads: finite, exact zeros on rows without an allowed pair, LSE -inf
    exactly on the queries without an allowed key."""
    q_ok, k_ok = row_has_pair(qo, ko)
    qd, kd = torch.from_numpy(q_ok).cuda(), torch.from_numpy(k_ok).cuda()
    for name, live in (("o", qd), ("dq", qd), ("dk", kd), ("dv", kd)):
        t = got[name]
        assert bool(torch.isfinite(t).all()), f"{name}: non-finite values"
        assert bool((t[~live] == 0).all()), f"{name}: rows without an allowed pair are not zero"
    lse = got["lse"]
    H = lse.shape[0]
    assert torch.equal(torch.isneginf(lse), (~qd)[None, :].expand(H, -1)), "LSE -inf pattern"
    assert bool(torch.isfinite(lse[:, qd]).all())
    return q_ok, k_ok


def _oracle_head(got, q, k, v, do, qo, ko, scale, h, q_ok, k_ok):
    """Head h against the fp64 oracle run on that head's slices alone."""
    sl = lambda a: np.ascontiguousarray(a[:, h:h + 1])  # noqa: E731
    ref = oatt.forward_backward(sl(q), sl(k), sl(v), sl(do), qo, ko, scale)
    res = {}
    for name, live in (("o", q_ok), ("dq", q_ok), ("dk", k_ok), ("dv", k_ok)):
        g = host64(got[name][:, h:h + 1])
        res[name] = compare(f"{name}[h={h}]", g, ref[name], live, "bf16")
    compare_lse(got["lse"][h:h + 1].cpu().numpy().astype(np.float64), ref["lse"])
    return res


def _full(pa, s, heads):
    print(f"[full] {s.name} nq={s.nq} nkv={s.nkv} oracle heads {heads}", flush=True)
    q, k, v, do = wl.make_values(s)
    (qo, ko), (qg, kg) = _ids(pa, s)
    got = _run(pa, _bf16(q), _bf16(k), _bf16(v), _bf16(do), qg, kg, s.scale)
    q_ok, k_ok = _device_checks(got, qo, ko)
    for h in heads:
        _oracle_head(got, q, k, v, do, qo, ko, s.scale, h, q_ok, k_ok)


def test_var_4x288_all_heads(pa):
    _full(pa, wl.config(3), range(24))


def test_equal_4x120_all_heads(pa):
    _full(pa, wl.config(2), range(24))


def test_long_mixed_64k(pa):
    _full(pa, wl.config(5), [0, 7, 11, 23])


def test_scattered_4x288(pa):
    """The 4 x 288 pack's segments cut into 512-token pieces and permuted: every
    tile's key list spans the sequence (the walk visits listed tiles only)."""
    _full(pa, wl.scattered_pack(), [0, 9, 17, 23])


@pytest.fixture(scope="module")
def sweep():
    """Both sweeps (self, cross) and one set of device values serving every batch."""
    self_b, cross_b = wl.bucketed_sweep(), wl.bucketed_sweep(cross=True)
    n_kv = max(s.nkv for s in self_b)
    n_q = max(max(s.nq for s in self_b), max(s.nq for s in cross_b))
    vals = wl.make_sweep_values(n_q, n_kv, 24, 128)
    dev = tuple(_bf16(a) for a in vals)
    return self_b, cross_b, vals, dev


SWEEP_CHUNKS = [(c, i0) for c in (False, True) for i0 in range(0, 40, 10)]


@pytest.mark.parametrize("cross,i0", SWEEP_CHUNKS)
def test_bucketed_sweep(pa, sweep, cross, i0):
    self_b, cross_b, (q, k, v, do), (Q, K, V, DO) = sweep
    batches = cross_b if cross else self_b
    assert len(batches) == 40
    for i in range(i0, i0 + 10):
        s = batches[i]
        h = (i + (12 if cross else 0)) % 24
        print(f"[sweep] {s.name} nq={s.nq} nkv={s.nkv} oracle head {h}", flush=True)
        (qo, ko), (qg, kg) = _ids(pa, s)
        got = _run(pa, Q[:s.nq], K[:s.nkv], V[:s.nkv], DO[:s.nq], qg, kg, s.scale)
        q_ok, k_ok = _device_checks(got, qo, ko)
        _oracle_head(got, q[:s.nq], k[:s.nkv], v[:s.nkv], do[:s.nq], qo, ko, s.scale, h, q_ok,
                     k_ok)
        del got
