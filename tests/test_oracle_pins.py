"""Pins of the CPU oracle against things other than itself.

* seq ids: hand-worked fixtures and closed-form counts.
* block mask: brute-force per-pair counting, hand-derived closed-form totals.
* attention: brute-force dense masked attention over the whole pack, torch's
  fp64 scaled_dot_product_attention with autograd per episode, central finite
  differences, closed forms (one-token episode, zero queries) and the pages'
  invariants (packed == per episode, padding rows exactly zero, no leakage
  across episodes, finite values, permutation equivariance).
"""
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import blockmask as obm
from oracle import seqids as osid
import workloads as wl


# ----------------------------------------------------------------- helpers
def _read_seq_fixture(path):
    cases, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {}
            cases.append(cur)
        else:
            cur[key] = [int(x) for x in vals]
    return cases


def _random_pack(rng, n, n_ids, d=16, h=2, neg_frac=0.2, interleave=True):
    ids = rng.integers(0, n_ids, n).astype(np.int32)
    ids[rng.random(n) < neg_frac] = -1
    if not interleave:
        ids = np.sort(ids)
    q = rng.standard_normal((n, h, d))
    k = rng.standard_normal((n, h, d))
    v = rng.standard_normal((n, h, d))
    do = rng.standard_normal((n, h, d))
    return ids, q, k, v, do


def _dense_masked(q, k, v, do, qid, kid, scale):
    """Brute force over the whole N x N score matrix with an explicit mask."""
    nq, h, d = q.shape
    out = {n: np.zeros_like(a) for n, a in (("o", q), ("dq", q), ("dk", k), ("dv", v))}
    lse = np.full((h, nq), -np.inf)
    allowed = (qid[:, None] == kid[None, :]) & (qid[:, None] >= 0)
    has = allowed.any(axis=1)
    for hh in range(h):
        S = scale * q[:, hh] @ k[:, hh].T
        Sm = np.where(allowed, S, -np.inf)
        m = np.where(has, Sm.max(axis=1), 0.0)
        e = np.where(allowed, np.exp(Sm - m[:, None]), 0.0)
        l = e.sum(axis=1)
        P = np.where(has[:, None], e / np.where(has, l, 1.0)[:, None], 0.0)
        lse[hh] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
        out["o"][:, hh] = P @ v[:, hh]
        dP = do[:, hh] @ v[:, hh].T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        out["dq"][:, hh] = scale * dS @ k[:, hh]
        out["dk"][:, hh] = scale * dS.T @ q[:, hh]
        out["dv"][:, hh] = P.T @ do[:, hh]
    out["lse"] = lse
    return out


def _close(a, b, rtol):
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() <= rtol * scale


# ----------------------------------------------------------------- seq ids
def test_seq_ids_hand_worked_fixture(golden_dir):
    for case in _read_seq_fixture(os.path.join(golden_dir, "seq_ids_small.txt")):
        got = osid.seq_ids_from_valid_frames(case["valid_frames"], case["frames_padded"][0],
                                             case["tokens_per_frame"][0])
        assert got.tolist() == case["ids"]


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_seq_ids_closed_form_counts(cfg):
    s = wl.config(cfg)
    ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    per_ep = s.frames_padded * s.q_tokens_per_frame
    assert len(ids) == s.nq
    for b, vf in enumerate(s.valid_frames):
        seg = ids[b * per_ep:(b + 1) * per_ep]
        n_valid = int(vf) * s.q_tokens_per_frame
        assert (seg[:n_valid] == b).all() and (seg[n_valid:] == -1).all()
    if cfg == 3:
        # 36,864 tokens of which 32*(119+177+285+239) = 26,240 are valid
        assert len(ids) == 36864 and int((ids >= 0).sum()) == 26240


# ----------------------------------------------------------------- block mask
def _brute_counts(qid, kid, bq, bkv):
    nqt, nkt = -(-len(qid) // bq), -(-len(kid) // bkv)
    cnt = np.zeros((nqt, nkt), np.int64)
    for i, a in enumerate(qid.tolist()):
        if a < 0:
            continue
        for j, b in enumerate(kid.tolist()):
            if a == b:
                cnt[i // bq, j // bkv] += 1
    return cnt


@pytest.mark.parametrize("seed", range(6))
def test_blockmask_counts_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    nq, nkv = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    nid = int(rng.integers(1, 6))
    qid = rng.integers(-2, nid, nq).astype(np.int32)
    kid = rng.integers(-2, nid, nkv).astype(np.int32)
    if seed % 2:
        qid.sort()
        kid.sort()
    for bq, bkv in ((16, 16), (32, 64), (64, 16), (128, 128)):
        cnt = obm.tile_pair_counts(qid, kid, bq, bkv)
        assert np.array_equal(cnt, _brute_counts(qid, kid, bq, bkv))
        cls = obm.tile_classes(qid, kid, bq, bkv)
        # full requires every position of a complete tile to be an allowed pair
        for i in range(cls.shape[0]):
            for j in range(cls.shape[1]):
                qs, ks = qid[i * bq:(i + 1) * bq], kid[j * bkv:(j + 1) * bkv]
                ok = (qs[:, None] == ks[None, :]) & (qs[:, None] >= 0)
                want = 0 if not ok.any() else (2 if (ok.all() and ok.size == bq * bkv) else 1)
                assert cls[i, j] == want


def test_blockmask_csr_lists_ascending_and_complete():
    rng = np.random.default_rng(7)
    qid = rng.integers(-1, 4, 700).astype(np.int32)
    kid = rng.integers(-1, 4, 500).astype(np.int32)
    cls = obm.tile_classes(qid, kid, 64, 32)
    q_ptr, q_cols, kv_ptr, kv_rows = obm.csr_lists(cls)
    for i in range(cls.shape[0]):
        row = q_cols[q_ptr[i]:q_ptr[i + 1]]
        assert row.tolist() == [j for j in range(cls.shape[1]) if cls[i, j]]
    for j in range(cls.shape[1]):
        col = kv_rows[kv_ptr[j]:kv_ptr[j + 1]]
        assert col.tolist() == [i for i in range(cls.shape[0]) if cls[i, j]]


def _golden_totals(golden_dir):
    rows = []
    for line in open(os.path.join(golden_dir, "tile_class_totals.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            n, bq, bkv, e, p, f = line.split()
            rows.append((n, int(bq), int(bkv), (int(e), int(p), int(f))))
    return rows


def test_blockmask_order_and_pair_lists_hand_worked():
    """Orders and pair walks of a hand-made class matrix (3 query x 4 key tiles):
    row lengths 2, 3, 2 -> query order 1, 0, 2 (ties by index); key-tile column
    lengths 2, 2, 1, 2 -> key order 0, 1, 3, 2.  Pair 0 = tiles (1, 0): union of
    {0, 1, 3} and {0, 2} = 0, 1, 2, 3; pair 1 = tile 2 alone: {1, 3}."""
    cls = np.array([[2, 0, 1, 0],
                    [1, 2, 0, 1],
                    [0, 1, 0, 2]], dtype=np.uint8)
    assert obm.longest_first_order(cls, 0).tolist() == [1, 0, 2]
    assert obm.longest_first_order(cls, 1).tolist() == [0, 1, 3, 2]
    room, lists = obm.pair_lists(cls, np.array([1, 0, 2]))
    assert room.tolist() == [0, 5, 7]
    e = lambda kt, a, b: kt | (a << 16) | (b << 24)  # noqa: E731
    assert lists[0].tolist() == [e(0, 1, 2), e(1, 2, 0), e(2, 0, 1), e(3, 1, 0)]
    assert lists[1].tolist() == [e(1, 1, 0), e(3, 2, 0)]


def test_blockmask_pair_lists_cover_both_lists(seed=7):
    """Each pair's walk is exactly the sorted union of its two tiles' CSR lists,
    and the classes beside each entry are the class matrix entries."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        nqt, nkt = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        cls = rng.choice(np.array([0, 0, 1, 2], np.uint8), size=(nqt, nkt))
        order = obm.longest_first_order(cls, 0)
        q_ptr, q_cols, _, _ = obm.csr_lists(cls)
        room, lists = obm.pair_lists(cls, order)
        for w, x in enumerate(lists):
            tiles = [int(order[2 * w])] + ([int(order[2 * w + 1])] if 2 * w + 1 < nqt else [])
            union = sorted(set().union(*[q_cols[q_ptr[t]:q_ptr[t + 1]].tolist() for t in tiles]))
            assert [v & 0xFFFF for v in x.tolist()] == union
            for v in x.tolist():
                kt = v & 0xFFFF
                assert (v >> 16) & 0xFF == cls[tiles[0], kt]
                assert (v >> 24) & 0xFF == (cls[tiles[1], kt] if len(tiles) > 1 else 0)
            assert room[w + 1] - room[w] == sum(q_ptr[t + 1] - q_ptr[t] for t in tiles)


def test_blockmask_closed_form_totals(golden_dir):
    by_name = {wl.config(i).name: wl.config(i) for i in (1, 2, 3)}
    for name, bq, bkv, want in _golden_totals(golden_dir):
        s = by_name[name]
        ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
        assert obm.class_totals(obm.tile_classes(ids, ids, bq, bkv)) == want, (name, bq, bkv)


# ----------------------------------------------------------------- attention
@pytest.mark.parametrize("seed", range(4))
def test_attention_matches_dense_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 150
    ids, q, k, v, do = _random_pack(rng, n, n_ids=4, interleave=bool(seed % 2))
    scale = 0.37
    got = oatt.forward_backward(q, k, v, do, ids, ids, scale, row_chunk=17)
    ref = _dense_masked(q, k, v, do, ids, ids, scale)
    for name in ("o", "dq", "dk", "dv"):
        assert _close(got[name], ref[name], 1e-12), name
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(fin, np.isfinite(got["lse"]))
    assert np.allclose(got["lse"][fin], ref["lse"][fin], rtol=1e-12, atol=1e-12)


def test_attention_cross_matches_dense_brute_force():
    rng = np.random.default_rng(11)
    nq, nkv, h, d = 70, 130, 2, 8
    qid = rng.integers(-1, 5, nq).astype(np.int32)
    kid = rng.integers(-1, 4, nkv).astype(np.int32)   # id 4 has queries but no keys
    q, do = rng.standard_normal((nq, h, d)), rng.standard_normal((nq, h, d))
    k, v = rng.standard_normal((nkv, h, d)), rng.standard_normal((nkv, h, d))
    got = oatt.forward_backward(q, k, v, do, qid, kid, 0.5)
    ref = _dense_masked(q, k, v, do, qid, kid, 0.5)
    for name in ("o", "dq", "dk", "dv"):
        assert _close(got[name], ref[name], 1e-12), name
    assert (got["o"][qid == 4] == 0).all() and np.isneginf(got["lse"][:, qid == 4]).all()


def test_attention_matches_torch_sdpa_autograd():
    s = wl.config(1)
    q, k, v, do = (a.astype(np.float64) for a in wl.make_values(s))
    ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    got = oatt.forward_backward(q, k, v, do, ids, ids, s.scale)
    for e in sorted(set(ids[ids >= 0].tolist())):
        r = np.flatnonzero(ids == e)
        for h in range(s.heads):
            Q, K, V = (torch.tensor(a[r, h], requires_grad=True) for a in (q, k, v))
            O = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None],
                                                                 scale=s.scale)[0]
            O.backward(torch.tensor(do[r, h]))
            np.testing.assert_allclose(got["o"][r, h], O.detach().numpy(), rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(got["dq"][r, h], Q.grad.numpy(), rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(got["dk"][r, h], K.grad.numpy(), rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(got["dv"][r, h], V.grad.numpy(), rtol=1e-9, atol=1e-12)


def test_attention_gradients_by_finite_differences():
    s = wl.config(1)
    q, k, v, do = (a.astype(np.float64) for a in wl.make_values(s))
    ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    got = oatt.forward_backward(q, k, v, do, ids, ids, s.scale)

    def loss(qq, kk, vv):
        o, _ = oatt.forward(qq, kk, vv, ids, ids, s.scale)
        return float((o * do).sum())

    rng = np.random.default_rng(5)
    eps = 1e-6
    for which, name in ((0, "dq"), (1, "dk"), (2, "dv")):
        for _ in range(50):
            i = int(rng.integers(0, s.nq))
            dd = int(rng.integers(0, s.head_dim))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][i, 0, dd] += eps
            lp = loss(*args)
            args[which][i, 0, dd] -= 2 * eps
            lm = loss(*args)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - got[name][i, 0, dd]) <= 1e-6 * (1 + abs(fd)), (name, i, dd)


def test_attention_closed_forms():
    rng = np.random.default_rng(3)
    h, d = 2, 8
    # episode 0 has one token; episode 1 has zero queries (uniform softmax)
    ids = np.array([0, 1, 1, 1, 1, -1], np.int32)
    q = rng.standard_normal((6, h, d))
    q[ids == 1] = 0.0
    k, v, do = (rng.standard_normal((6, h, d)) for _ in range(3))
    r = oatt.forward_backward(q, k, v, do, ids, ids, 0.25)
    assert np.allclose(r["o"][0], v[0], rtol=0, atol=1e-15)
    assert np.abs(r["dq"][0]).max() < 1e-15 and np.abs(r["dk"][0]).max() < 1e-15
    assert np.allclose(r["dv"][0], do[0], rtol=0, atol=1e-15)
    ep1 = ids == 1
    for hh in range(h):
        assert np.allclose(r["o"][ep1, hh], v[ep1, hh].mean(axis=0)[None], atol=1e-14)
        assert np.allclose(r["lse"][hh, ep1], np.log(4.0), atol=1e-14)
        # uniform P: dV_j = (1/4) sum_i dO_i
        assert np.allclose(r["dv"][ep1, hh], do[ep1, hh].sum(axis=0)[None] / 4, atol=1e-14)
    assert (r["o"][5] == 0).all() and (r["dq"][5] == 0).all()
    assert (r["dk"][5] == 0).all() and (r["dv"][5] == 0).all()
    assert np.isneginf(r["lse"][:, 5]).all()


def test_single_unpadded_episode_is_plain_softmax_attention():
    rng = np.random.default_rng(9)
    n, d = 40, 16
    q, k, v = (rng.standard_normal((n, 1, d)) for _ in range(3))
    ids = np.zeros(n, np.int32)
    o, lse = oatt.forward(q, k, v, ids, ids, 0.25)
    S = 0.25 * q[:, 0] @ k[:, 0].T
    P = np.exp(S) / np.exp(S).sum(axis=1, keepdims=True)
    assert np.allclose(o[:, 0], P @ v[:, 0], rtol=1e-13, atol=1e-14)
    assert np.allclose(lse[0], np.log(np.exp(S).sum(axis=1)), rtol=1e-13)


def test_invariants_packed_equals_per_episode_and_no_leakage():
    s = wl.config(1)
    q, k, v, do = (a.astype(np.float64) for a in wl.make_values(s))
    ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    full = oatt.forward_backward(q, k, v, do, ids, ids, s.scale)
    for name in ("o", "dq", "dk", "dv", "lse"):
        assert np.isfinite(full[name][..., ids >= 0] if name == "lse" else full[name]).all()
    # padding rows are exactly zero, and their LSE is -inf
    pad = ids < 0
    for name in ("o", "dq", "dk", "dv"):
        assert (full[name][pad] == 0).all()
    assert np.isneginf(full["lse"][:, pad]).all()
    # each episode run alone gives the same rows
    for e in range(s.n_episodes):
        r = np.flatnonzero(ids == e)
        one = oatt.forward_backward(q[r], k[r], v[r], do[r], ids[r], ids[r], s.scale)
        for name in ("o", "dq", "dk", "dv"):
            assert np.array_equal(one[name], full[name][r]), (e, name)
    # perturbing episode 1 leaves episodes 0 and 2 bit-identical
    r1 = ids == 1
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    for a in (q2, k2, v2, do2):
        a[r1] += 1.0
    pert = oatt.forward_backward(q2, k2, v2, do2, ids, ids, s.scale)
    other = ~r1
    for name in ("o", "dq", "dk", "dv"):
        assert np.array_equal(pert[name][other], full[name][other])
        assert not np.array_equal(pert[name][r1], full[name][r1])


def test_invariants_relabel_and_permute():
    rng = np.random.default_rng(21)
    ids, q, k, v, do = _random_pack(rng, 120, n_ids=5)
    base = oatt.forward_backward(q, k, v, do, ids, ids, 0.3)
    relabel = np.where(ids >= 0, 1000 - 7 * ids, -5).astype(np.int32)
    rl = oatt.forward_backward(q, k, v, do, relabel, relabel, 0.3)
    for name in ("o", "dq", "dk", "dv"):
        assert np.allclose(rl[name], base[name], rtol=1e-13, atol=1e-13)
    p = rng.permutation(len(ids))
    pm = oatt.forward_backward(q[p], k[p], v[p], do[p], ids[p], ids[p], 0.3)
    for name in ("o", "dq", "dk", "dv"):
        assert np.allclose(pm[name], base[name][p], rtol=1e-12, atol=1e-12)


def test_head_subset_matches_all_heads():
    rng = np.random.default_rng(4)
    ids, q, k, v, do = _random_pack(rng, 90, n_ids=3, h=3)
    full = oatt.forward_backward(q, k, v, do, ids, ids, 0.3)
    sub = oatt.forward_backward(q, k, v, do, ids, ids, 0.3, heads=[2])
    for name in ("o", "dq", "dk", "dv"):
        assert np.array_equal(sub[name][:, 2], full[name][:, 2])
        assert np.isnan(sub[name][:, 0]).all()


def test_useful_pairs_closed_form():
    s = wl.config(3)
    ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    # sum over episodes of (32 * frames)^2
    assert oatt.useful_pairs(ids, ids) == sum((32 * int(f)) ** 2 for f in (119, 177, 285, 239))
    assert oatt.useful_pairs(ids, ids) == 188248064


# ----------------------------------------------------------------- unpadded packing
def _read_unpadded_fixture(path):
    cases = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, rest = line.split(None, 1) if " " in line else (line, "")
        a, b, c = (x.strip() for x in rest.split("|"))
        lengths = [int(x) for x in a.split(",")] if a else []
        if kind == "ids":
            cases.append(("ids", lengths, int(b), [int(x) for x in c.split(",")]))
        else:
            cases.append(("packs", lengths, int(b),
                          [[int(x) for x in p.split(",")] for p in c.split(";")]))
    return cases


def test_unpadded_hand_worked_fixture(golden_dir):
    from oracle import packing as opk
    cases = _read_unpadded_fixture(os.path.join(golden_dir, "unpadded_packs_small.txt"))
    assert len(cases) == 7
    for kind, lengths, n, want in cases:
        if kind == "ids":
            assert osid.seq_ids_from_lengths(lengths, n).tolist() == want, (lengths, n)
        else:
            assert opk.next_fit_packs(lengths, n) == want, (lengths, n)


@pytest.mark.parametrize("seed", range(5))
def test_unpadded_ids_equal_repeat_construction(seed):
    """Same ids as numpy's repeat of the episode index, cut / padded to length."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(-3, 40, int(rng.integers(0, 12)))
    n = int(rng.integers(1, 300))
    rep = np.repeat(np.arange(len(lengths), dtype=np.int32), np.maximum(lengths, 0))
    want = np.full(n, -1, np.int32)
    want[:min(n, len(rep))] = rep[:n]
    assert np.array_equal(osid.seq_ids_from_lengths(lengths, n), want)


@pytest.mark.parametrize("seed", range(8))
def test_next_fit_is_the_unique_order_preserving_maximal_partition(seed):
    """Next-fit is characterised by: packs are consecutive runs of the input
    order, each within the budget, and each pack's first episode would not
    have fit in the pack before it.  Check those three properties."""
    from oracle import packing as opk
    rng = np.random.default_rng(seed)
    budget = int(rng.integers(5, 60))
    lengths = rng.integers(0, budget + 1, int(rng.integers(1, 40))).tolist()
    packs = opk.next_fit_packs(lengths, budget)
    assert [e for p in packs for e in p] == list(range(len(lengths)))
    sums = [sum(lengths[e] for e in p) for p in packs]
    assert all(s <= budget for s in sums) and all(len(p) > 0 for p in packs)
    for k in range(1, len(packs)):
        assert sums[k - 1] + lengths[packs[k][0]] > budget


def test_next_fit_rejects_an_episode_over_budget():
    from oracle import packing as opk
    with pytest.raises(ValueError):
        opk.next_fit_packs([3, 11, 2], 10)
