"""The no-allocation backward entry point (attn_packed_bwd_noalloc), called
through the C ABI, against the workspace-taking attn_packed_bwd (the same
kernels: bit-identical gradients) and the fp64 oracle (the stated tolerance),
on two calls in a row, the second on a smaller pack, so that the fixed array
holds the first call's row terms when the second starts."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oatt
from oracle import seqids as osid
from tests._helpers import compare, compare_lse, host64, ids_dev, row_has_pair, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return pa_mod


def _spec(valid, fp, tq, tk, heads, d, dtype, seed):
    return wl.PackSpec(f"noalloc-{seed}", heads=heads, head_dim=d, dtype=dtype, seed=seed,
                       value_std=0.5 if dtype == "bf16" else 1.0,
                       valid_frames=np.array(valid, np.int32), frames_padded=fp,
                       q_tokens_per_frame=tq, kv_tokens_per_frame=tk)


def _one_call(pa, s):
    q, k, v, do = wl.make_values(s)
    qo = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    ko = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.kv_tokens_per_frame)
    vf = ids_dev(s.valid_frames)
    qg = pa.seq_ids_from_valid_frames(vf, s.frames_padded, s.q_tokens_per_frame)
    kg = pa.seq_ids_from_valid_frames(vf, s.frames_padded, s.kv_tokens_per_frame)
    Q, K, V, DO = (to_dev(a, s.dtype) for a in (q, k, v, do))
    mask = pa.build_block_mask(qg, kg, 128, 128)
    o, lse = pa.attn_packed_fwd(Q, K, V, qg, kg, mask, s.scale)
    nan = float("nan")
    grads = tuple(torch.full_like(t, nan) for t in (Q, K, V))  # every row must be written
    pa.attn_packed_bwd_noalloc(Q, K, V, o, DO, lse, qg, kg, mask, s.scale, grads=grads)
    ref_ws = pa.attn_packed_bwd(Q, K, V, o, DO, lse, qg, kg, mask, s.scale)
    torch.cuda.synchronize()
    for a, b in zip(grads, ref_ws):
        assert torch.equal(a, b)
    ref = oatt.forward_backward(q, k, v, do, qo, ko, s.scale)
    q_ok, k_ok = row_has_pair(qo, ko)
    compare("dQ", host64(grads[0]), ref["dq"], q_ok, s.dtype)
    compare("dK", host64(grads[1]), ref["dk"], k_ok, s.dtype)
    compare("dV", host64(grads[2]), ref["dv"], k_ok, s.dtype)
    compare_lse(lse.cpu().numpy().astype(np.float64), ref["lse"])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_noalloc_backward_two_calls(pa, dtype, d):
    print(f"[noalloc] {dtype} d={d}", flush=True)
    assert pa.attn_packed_bwd_noalloc_max_bytes() == 64 << 20
    _one_call(pa, _spec([5, 9, 0, 3, 7], 9, 32, 32, 8, d, dtype, 41))   # 1,440 tokens, 8 heads
    _one_call(pa, _spec([3, 2], 5, 16, 16, 3, d, dtype, 42))            # then 160 tokens, 3 heads

