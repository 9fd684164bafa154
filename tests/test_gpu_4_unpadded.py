"""GPU parity of unpadded packing: ids from episode lengths (bit-exact against
the oracle, with the episode offsets), and packed attention fwd+bwd on a full
68,000-token unpadded pack planned by the library's next-fit packer.
Attention tolerances: tests/_helpers.py (bf16)."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oatt
from oracle import packing as opk
from oracle import seqids as osid
from tests._helpers import compare, compare_lse, host64, ids_dev, row_has_pair, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return pa_mod


def _ids_case(pa, lengths, n):
    print(f"ids case B={len(lengths)} n={n}", flush=True)
    L = torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    ids, off = pa.seq_ids_from_lengths(L, n, offsets=True)
    torch.cuda.synchronize()
    want = osid.seq_ids_from_lengths(lengths, n)
    assert np.array_equal(ids.cpu().numpy(), want)
    # offsets: where each episode starts in the buffer and how many tokens carry an id
    ends = np.minimum(np.cumsum(np.maximum(np.asarray(lengths, np.int64), 0)), n)
    starts = np.concatenate([[0], ends[:-1]]) if len(lengths) else np.zeros(0, np.int64)
    want_off = np.concatenate([starts, [ends[-1] if len(lengths) else 0]])
    assert np.array_equal(off.cpu().numpy(), want_off.astype(np.int32))


@pytest.mark.parametrize("seed", range(4))
def test_ids_random(pa, seed):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(-5, 3000, int(rng.integers(1, 40)))
    lengths[rng.integers(0, len(lengths), 3)] = 0
    n = int(max(1, rng.integers(0, int(np.maximum(lengths, 0).sum()) + 2000)))
    _ids_case(pa, lengths, n)


def test_ids_edge_cases(pa):
    _ids_case(pa, [3, 0, 2], 8)
    _ids_case(pa, [4, 5], 6)                      # cut at the buffer end
    _ids_case(pa, [], 5)                          # nothing placed: all -1
    _ids_case(pa, [0, 0, 7], 7)                   # exact fill after empty episodes
    _ids_case(pa, [1] * 8192, 9000)               # the maximum episode count
    _ids_case(pa, [2**31 - 1, 5], 4099)           # huge length, 64-bit prefix sums
    L = torch.tensor([3, 4], dtype=torch.int32, device="cuda")
    _, off = pa.seq_ids_from_lengths(L, 0, offsets=True)   # empty buffer, offsets only
    assert off.cpu().tolist() == [0, 0, 0]


def test_unpadded_68k_pack_attention(pa):
    lengths = wl.episode_stream()
    pack_of, n_packs = pa.plan_token_packs(lengths, wl.UNPADDED_BUDGET)
    packs = opk.next_fit_packs(lengths, wl.UNPADDED_BUDGET)
    assert n_packs == len(packs) and [int(pack_of[p[0]]) for p in packs] == list(range(n_packs))
    sel = lengths[pack_of == 0]
    assert sel.tolist() == [int(lengths[e]) for e in packs[0]]
    s = wl.unpadded_pack(sel)
    heads = [0, 13]
    print(f"unpadded pack: {len(sel)} episodes, {int(sel.sum())} of {s.nq} tokens; "
          f"heads {heads}", flush=True)
    q, k, v, do = wl.make_values(s)
    ids = pa.seq_ids_from_lengths(torch.from_numpy(sel).cuda(), s.nq)
    oid = osid.seq_ids_from_lengths(sel, s.nq)
    assert np.array_equal(ids.cpu().numpy(), oid)
    Q, K, V, DO = (to_dev(a, "bf16") for a in (q, k, v, do))
    mask = pa.build_block_mask(ids, ids, 128, 128)
    o, lse = pa.attn_packed_fwd(Q, K, V, ids, ids, mask, s.scale)
    dq, dk, dv = pa.attn_packed_bwd(Q, K, V, o, DO, lse, ids, ids, mask, s.scale)
    torch.cuda.synchronize()
    got = dict(o=host64(o), lse=lse.cpu().numpy().astype(np.float64), dq=host64(dq),
               dk=host64(dk), dv=host64(dv))
    ref = oatt.forward_backward(q, k, v, do, oid, oid, s.scale, heads=heads)
    live, _ = row_has_pair(oid, oid)
    for name in ("o", "dq", "dk", "dv"):
        compare(name, got[name], ref[name], live, "bf16", heads)
        g = got[name]
        assert np.isfinite(g).all() and (g[~live] == 0).all()   # every head: dead rows zero
    compare_lse(got["lse"], ref["lse"], heads)
