"""Host batch planning in the C library (length_bucket_batches,
dual_constraint_batch, fit_step_cost) against the oracle; no GPU needed.
Batches must match exactly; the cost fit within 1e-6 in p and 1e-4 relative
in a and b (two independent one-dimensional minimisers)."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import sampler as osm


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    return pa_mod


def _frames():
    return (wl.episode_stream() // 32).tolist()


@pytest.mark.parametrize("seed,epoch,pool,bs", [(7, 0, 200, 4), (7, 3, 200, 4), (11, 1, 24, 3),
                                                (0, 0, 1, 1), (5, 2, 1000, 7)])
def test_fixed_batches_match_oracle(pa, seed, epoch, pool, bs):
    fr = _frames()
    got = pa.length_bucket_batches(fr, seed, epoch, pool, 8, bs)
    want = osm.length_bucket_batches(fr, seed=seed, epoch=epoch, pool_size=pool, pad_multiple=8,
                                     batch_size=bs)
    assert got == (want[0], want[1])


@pytest.mark.parametrize("world", [2, 3, 8])
def test_rank_shards_match_oracle(pa, world):
    fr = _frames()[:149]
    for r in range(world):
        got = pa.length_bucket_batches(fr, 9, 1, 30, 8, 4, rank=r, world_size=world)
        want = osm.length_bucket_batches(fr, seed=9, epoch=1, pool_size=30, pad_multiple=8,
                                         batch_size=4, rank=r, world_size=world)
        assert got == (want[0], want[1])


@pytest.mark.parametrize("m_comp,p", [(4e8, 2.0), (1.5e8, 1.8), (1e12, 2.2)])
def test_dual_constraint_batches_match_oracle(pa, m_comp, p):
    fr = _frames()
    dual = (68000.0, m_comp, p, 32)
    got = pa.length_bucket_batches(fr, 3, 0, 50, 8, 0, dual=dual)
    want = osm.length_bucket_batches(fr, seed=3, epoch=0, pool_size=50, pad_multiple=8,
                                     dual=dual)
    assert got == (want[0], want[1])


def test_dual_constraint_batch_values(pa):
    for s in (1000, 3296, 9216, 11584, 100000):
        for m_comp, p in ((4e8, 2.0), (3e7, 1.7), (1e15, 2.5)):
            assert pa.dual_constraint_batch(s, 68000, m_comp, p) == \
                osm.dual_constraint_batch(s, 68000, m_comp, p)


def test_fit_matches_oracle(pa):
    rng = np.random.default_rng(0)
    B = np.array([1, 2, 4, 8, 1, 2, 4, 1, 2, 1, 3, 5], float)
    S = np.array([2048, 2048, 2048, 2048, 4096, 4096, 4096, 8192, 8192, 16384, 6000, 3000], float)
    t = 0.2 + 3e-8 * B * S ** 1.9 * (1 + 0.02 * rng.standard_normal(len(B)))
    a, b, p = pa.fit_step_cost(B, S, t)
    oa, ob, op = osm.fit_step_cost(B, S, t)
    assert abs(p - op) < 1e-6
    assert math.isclose(a, oa, rel_tol=1e-4, abs_tol=1e-9) and math.isclose(b, ob, rel_tol=1e-4)


def test_planner_argument_errors(pa):
    lib = pa.packattn._lib
    assert lib.dual_constraint_batch(0.0, 1.0, 1.0, 2.0) == -2
    assert lib.dual_constraint_batch(10.0, -1.0, 1.0, 2.0) == -2
    assert lib.length_bucket_rank_size(10, 0) == 0
    with pytest.raises(pa.PackAttnError):
        pa.length_bucket_batches([3, 4], 0, 0, 0, 8, 4)          # pool_size 0
    with pytest.raises(pa.PackAttnError):
        pa.length_bucket_batches([3, 4], 0, 0, 4, 8, 4, rank=2, world_size=2)
    with pytest.raises(pa.PackAttnError):
        pa.length_bucket_batches([3, 4], 0, 0, 4, 8, 0)          # dual constraint missing
    with pytest.raises(pa.PackAttnError):
        pa.fit_step_cost([1.0], [2.0], [3.0])                     # one point
    assert pa.length_bucket_batches([], 0, 0, 4, 8, 4) == ([], [])
