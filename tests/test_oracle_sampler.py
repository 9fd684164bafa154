"""Pins of the sampler / planner oracle (oracle/sampler.py).

  * SplitMix64 reproduces the known-answer outputs of its reference
    implementation from state 0;
  * the shuffle is a permutation and is uniform over the 6 orders of 3 items
    (chi-square over 6000 seeds);
  * sampler invariants from the packing report, section 2.1: each episode
    once per epoch on one rank; with several ranks every rank has the same
    batch count and the ranks together cover every episode (tail repeats
    only); batches are length-sorted runs of their pool; padded frames are
    the batch maximum rounded up; the bucketing keeps padding waste on the
    160-episode stream under 10 % (the target the report sets);
  * the dual constraint (AdaptiveLoad summary, section 2A) by hand-worked
    values and a hand-cut pool; every dual-constraint batch is within its
    bound, and no batch could take the next episode of its sorted pool;
  * the cost fit recovers (a, b, p) from exact synthetic timings.
"""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import sampler as osm


def test_splitmix64_known_answers():
    g = osm.SplitMix64(0)
    assert [g.next() for _ in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                            0x06C45D188009454F]


def test_shuffle_is_a_uniform_permutation():
    counts = {}
    for seed in range(6000):
        p = tuple(osm.shuffle([0, 1, 2], osm.SplitMix64(seed)))
        counts[p] = counts.get(p, 0) + 1
    assert len(counts) == 6
    chi2 = sum((c - 1000) ** 2 / 1000 for c in counts.values())
    assert chi2 < 25.0                    # 5 degrees of freedom; p ~ 1e-4
    for n in (0, 1, 17):
        assert sorted(osm.shuffle(list(range(n)), osm.SplitMix64(3))) == list(range(n))


def _frames():
    return (wl.episode_stream() // 32).tolist()     # 160 episodes of 103..362 frames


def test_single_rank_invariants():
    fr = _frames()
    batches, fpad = osm.length_bucket_batches(fr, seed=7, epoch=0, pool_size=200,
                                              pad_multiple=8, batch_size=4)
    flat = [e for b in batches for e in b]
    assert sorted(flat) == list(range(len(fr)))
    assert all(len(b) == 4 for b in batches)
    for b, f in zip(batches, fpad):
        assert [fr[e] for e in b] == sorted(fr[e] for e in b)
        assert f == osm.round_up(max(fr[e] for e in b), 8) and f % 8 == 0
    real = sum(fr)
    padded = sum(f * len(b) for b, f in zip(batches, fpad))
    assert (padded - real) / padded < 0.10
    again, _ = osm.length_bucket_batches(fr, seed=7, epoch=0, pool_size=200, pad_multiple=8,
                                         batch_size=4)
    other, _ = osm.length_bucket_batches(fr, seed=7, epoch=1, pool_size=200, pad_multiple=8,
                                         batch_size=4)
    assert again == batches and other != batches


def test_multi_rank_sharding():
    fr = _frames()[:151]                  # not a multiple of the world size
    W = 4
    per = [osm.length_bucket_batches(fr, seed=1, epoch=2, pool_size=40, pad_multiple=8,
                                     batch_size=4, rank=r, world_size=W)[0] for r in range(W)]
    assert len({len(b) for b in per}) == 1
    seen = [e for bs in per for b in bs for e in b]
    assert len(seen) == 152 and set(seen) == set(range(151))


def test_dual_constraint_hand_worked():
    # S = 9216 tokens, memory 68000 tokens -> 7; compute 4e8 at p = 2 -> 4e8/84.9e6 = 4.7 -> 4
    assert osm.dual_constraint_batch(9216, 68000, 4e8, 2.0) == 4
    assert osm.dual_constraint_batch(3296, 68000, 4e8, 2.0) == 20
    assert osm.dual_constraint_batch(100000, 68000, 4e8, 2.0) == 1     # never below 1
    assert osm.dual_constraint_batch(1000, 68000, 1e12, 2.0) == 68     # memory binds


def test_dual_constraint_batches_are_within_bound_and_maximal():
    fr = _frames()
    dual = (68000.0, 4e8, 2.0, 32)
    batches, fpad = osm.length_bucket_batches(fr, seed=3, epoch=0, pool_size=50, pad_multiple=8,
                                              dual=dual)
    assert sorted(e for b in batches for e in b) == list(range(len(fr)))
    for b, f in zip(batches, fpad):
        s = f * 32
        assert len(b) == 1 or len(b) <= osm.dual_constraint_batch(s, *dual[:3])
    sizes = [len(b) for b in batches]
    assert min(sizes) >= 1 and max(sizes) > 4      # short episodes get bigger batches


def test_dual_constraint_cut_hand_worked_pool():
    """One pool, cut by hand (AdaptiveLoad summary, section 2A, bound per batch;
    32 tokens per frame, multiple of 8 frames, M_mem 68,000, M_comp 4e8, p 2):
      * 100 frames -> S = 104*32 = 3,328, bound min(20, floor(36.1)) = 20;
      * with a 200-frame episode S = 200*32 = 6,400, bound min(10, floor(9.77)) = 9:
        seven 100s and two 200s make 9 <= 9, a third 200 would make 10 > 9 -> cut;
      * the third 200 with the two 300s: S = 304*32 = 9,728, bound
        min(6, floor(4.23)) = 4, so 3 <= 4 -> one batch to the end of the pool.
    An off-by-one in the cut (closing a batch when it reaches the bound instead
    of when it would exceed it) gives 8 + 4 instead of 9 + 3."""
    frames = [100] * 7 + [200] * 3 + [300] * 2
    dual = (68000.0, 4e8, 2.0, 32)
    assert osm.dual_constraint_batch(3328, *dual[:3]) == 20
    assert osm.dual_constraint_batch(6400, *dual[:3]) == 9
    assert osm.dual_constraint_batch(9728, *dual[:3]) == 4
    batches, fpad = osm.length_bucket_batches(frames, seed=5, epoch=0, pool_size=len(frames),
                                              pad_multiple=8, dual=dual)
    got = sorted(([frames[e] for e in b], f) for b, f in zip(batches, fpad))
    assert got == [([100] * 7 + [200] * 2, 200), ([200, 300, 300], 304)]


def test_dual_constraint_batches_cannot_grow():
    """Maximality on the 160-episode stream, one pool: batches are consecutive
    runs of the sorted pool, so ordered by (smallest, largest) frame count each
    batch but the last would break its bound if it took the first episode of
    the next one."""
    fr = _frames()
    dual = (68000.0, 4e8, 2.0, 32)
    batches, _ = osm.length_bucket_batches(fr, seed=11, epoch=0, pool_size=len(fr),
                                           pad_multiple=8, dual=dual)
    runs = sorted(([fr[e] for e in b] for b in batches), key=lambda r: (min(r), max(r)))
    assert [x for r in runs for x in sorted(r)] == sorted(fr)
    for cur, nxt in zip(runs, runs[1:]):
        grown = cur + [min(nxt)]
        s = osm.round_up(max(grown), 8) * 32
        assert len(grown) > osm.dual_constraint_batch(s, *dual[:3])
        s_cur = osm.round_up(max(cur), 8) * 32
        assert len(cur) == 1 or len(cur) <= osm.dual_constraint_batch(s_cur, *dual[:3])


def test_cost_fit_recovers_exact_parameters():
    B = np.array([1, 2, 4, 8, 1, 2, 4, 1, 2, 1], float)
    S = np.array([2048, 2048, 2048, 2048, 4096, 4096, 4096, 8192, 8192, 16384], float)
    a, b, p = 0.3, 2.5e-8, 1.85
    t = a + b * B * S ** p
    fa, fb, fp = osm.fit_step_cost(B, S, t)
    assert abs(fp - p) < 1e-6 and math.isclose(fa, a, rel_tol=1e-5) \
        and math.isclose(fb, b, rel_tol=1e-5)
