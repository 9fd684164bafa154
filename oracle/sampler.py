"""Oracle: length-bucket batch sampler and dual-constraint batch sizing
(TEST INFRASTRUCTURE -- see ``oracle/__init__.py``).

"LingBot-VA packing" report, section 2.1 (LengthBucketBatchSampler and the pad
collate): every epoch the episode list is shuffled with seed + epoch, sharded
round-robin over the ranks with the tail padded so every rank gets the same
number of batches, cut into pools of batch_size * pool_factor episodes, each
pool sorted by length and cut into batches, and the batch order shuffled; a
batch is zero-padded to round_up(max frames, pad_multiple).

AdaptiveLoad summary, section 2A: a bucket of sequence length S gets the batch
size B = max(1, min(floor(M_mem / S), floor(M_comp / S^p))), from the linear
memory constraint B*S <= M_mem and the polynomial compute constraint
B*S^p <= M_comp; p and M_comp come from fitting step time ~ a + b*B*S^p to
measured shapes.

Readings taken where the pages leave a step open:
  * the shuffle generator is SplitMix64 (Steele, Lea and Flood, 2014) seeded
    with seed + epoch, and a Fisher-Yates shuffle drawing j in [0, i] as the
    high 64 bits of next() * (i + 1); the batch-order shuffle continues the
    same stream;
  * tail padding repeats the shuffled list from its start up to a multiple of
    world_size; rank r takes positions r, r + W, ...;
  * pools are consecutive runs of the rank's list; sorting is ascending and
    stable; a pool's last batch may be short;
  * with the dual constraint, a sorted pool is cut greedily: a batch grows
    while its size stays within B(S) of its padded sequence length
    S = round_up(max frames, pad_multiple) * tokens_per_frame;
  * the fit is least squares in the step time: for each p, a and b solve the
    linear problem exactly; p minimises the residual over [p_lo, p_hi].
"""
from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

MASK64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64: state += 0x9E3779B97F4A7C15, then the output mix."""

    def __init__(self, state: int):
        self.state = state & MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)

    def below(self, bound: int) -> int:
        """An integer in [0, bound): high 64 bits of next() * bound."""
        return (self.next() * bound) >> 64


def shuffle(items: list, gen: SplitMix64) -> list:
    """Fisher-Yates, from the last position down."""
    out = list(items)
    for i in range(len(out) - 1, 0, -1):
        j = gen.below(i + 1)
        out[i], out[j] = out[j], out[i]
    return out


def round_up(x: int, m: int) -> int:
    return (int(x) + m - 1) // m * m


def dual_constraint_batch(seq_len: float, m_mem: float, m_comp: float, p: float) -> int:
    """B = max(1, min(floor(M_mem / S), floor(M_comp / S^p)))."""
    return max(1, min(math.floor(m_mem / seq_len), math.floor(m_comp / seq_len ** p)))


def length_bucket_batches(frames, seed: int, epoch: int, pool_size: int, pad_multiple: int,
                          batch_size: int = 0, rank: int = 0, world_size: int = 1,
                          dual: Optional[Tuple[float, float, float, int]] = None):
    """Batches of one rank for one epoch: (list of index lists, padded frames).

    ``batch_size > 0`` cuts fixed batches; ``batch_size == 0`` uses the dual
    constraint ``dual = (m_mem, m_comp, p, tokens_per_frame)``.
    """
    n = len(frames)
    gen = SplitMix64(seed + epoch)
    order = shuffle(list(range(n)), gen)
    if n == 0:
        return [], []
    total = -(-n // world_size) * world_size
    padded = [order[i % n] for i in range(total)]
    mine = padded[rank::world_size]
    batches: List[List[int]] = []
    for p0 in range(0, len(mine), pool_size):
        pool = sorted(mine[p0:p0 + pool_size], key=lambda e: frames[e])  # stable
        if batch_size > 0:
            for b0 in range(0, len(pool), batch_size):
                batches.append(pool[b0:b0 + batch_size])
        else:
            m_mem, m_comp, pexp, tpf = dual
            cur: List[int] = []
            for e in pool:
                cand = cur + [e]
                s = round_up(max(frames[i] for i in cand), pad_multiple) * tpf
                if cur and len(cand) > dual_constraint_batch(s, m_mem, m_comp, pexp):
                    batches.append(cur)
                    cur = [e]
                else:
                    cur = cand
            if cur:
                batches.append(cur)
    batches = shuffle(batches, gen)
    fpad = [round_up(max(frames[i] for i in b), pad_multiple) for b in batches]
    return batches, fpad


def fit_step_cost(B, S, t, p_lo: float = 1.0, p_hi: float = 3.0):
    """Least-squares fit of t ~ a + b * B * S^p: returns (a, b, p)."""
    from scipy.optimize import minimize_scalar
    B, S, t = (np.asarray(v, dtype=np.float64) for v in (B, S, t))

    def solve(p):
        X = np.stack([np.ones_like(t), B * S ** p], axis=1)
        coef, *_ = np.linalg.lstsq(X, t, rcond=None)
        return coef, float(((X @ coef - t) ** 2).sum())

    res = minimize_scalar(lambda p: solve(p)[1], bounds=(p_lo, p_hi), method="bounded",
                          options={"xatol": 1e-10})
    (a, b), _ = solve(res.x)
    return float(a), float(b), float(res.x)
