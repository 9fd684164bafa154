"""Host-side unpadded packing (plan_token_packs in the C library) against the
next-fit oracle, and argument checks of seq_ids_from_lengths; no GPU needed."""
import ctypes

import numpy as np
import pytest

import workloads as wl
from oracle import packing as opk


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    return pa_mod


def _as_lists(pack_of, n):
    packs = [[] for _ in range(n)]
    for e, p in enumerate(pack_of.tolist()):
        packs[p].append(e)
    return packs


@pytest.mark.parametrize("seed", range(10))
def test_plan_matches_oracle_random(pa, seed):
    rng = np.random.default_rng(seed)
    budget = int(rng.integers(1, 100))
    lengths = rng.integers(0, budget + 1, int(rng.integers(0, 60)))
    pack_of, n = pa.plan_token_packs(lengths, budget)
    assert _as_lists(pack_of, n) == (opk.next_fit_packs(lengths, budget) if len(lengths) else [])


def test_plan_matches_oracle_on_the_episode_stream(pa):
    lengths = wl.episode_stream()
    pack_of, n = pa.plan_token_packs(lengths, wl.UNPADDED_BUDGET)
    want = opk.next_fit_packs(lengths, wl.UNPADDED_BUDGET)
    assert _as_lists(pack_of, n) == want
    fill = [sum(int(lengths[e]) for e in p) / wl.UNPADDED_BUDGET for p in want[:-1]]
    assert min(fill) > 0.8          # every closed pack is more than 80 % full
    sizes = [len(p) for p in want]
    assert 5 <= np.median(sizes) <= 12


def test_plan_errors(pa):
    lib = pa.packattn._lib
    n = ctypes.c_int32(0)
    out = (ctypes.c_int32 * 3)()
    arr = (ctypes.c_int32 * 3)(3, 11, 2)
    assert lib.plan_token_packs(arr, 3, 10, out, ctypes.byref(n)) == -2     # over budget
    arr2 = (ctypes.c_int32 * 3)(3, -1, 2)
    assert lib.plan_token_packs(arr2, 3, 10, out, ctypes.byref(n)) == -2    # negative length
    assert lib.plan_token_packs(arr, 3, 0, out, ctypes.byref(n)) == -2      # budget < 1
    assert lib.plan_token_packs(None, 3, 10, out, ctypes.byref(n)) == -1
    assert lib.plan_token_packs(arr, 3, 10, out, None) == -1
    assert lib.plan_token_packs(None, 0, 10, None, ctypes.byref(n)) == 0 and n.value == 0


def test_seq_ids_from_lengths_argument_errors(pa):
    lib = pa.packattn._lib
    fake = ctypes.c_void_p(0x100000)
    assert lib.seq_ids_from_lengths(fake, -1, 10, fake, None, None) == -2
    assert lib.seq_ids_from_lengths(fake, 8193, 10, fake, None, None) == -2   # > 8192 episodes
    assert lib.seq_ids_from_lengths(fake, 3, -5, fake, None, None) == -2
    assert lib.seq_ids_from_lengths(None, 3, 10, fake, None, None) == -1
    assert lib.seq_ids_from_lengths(fake, 3, 10, None, None, None) == -1
    assert lib.seq_ids_from_lengths(None, 0, 0, None, None, None) == 0       # nothing to do
