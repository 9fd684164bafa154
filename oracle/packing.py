"""Oracle: assigning episodes to unpadded packs under a token budget
(TEST INFRASTRUCTURE -- see ``oracle/__init__.py``).

"LingBot-VA packing" report, section 1: one episode per micro-step uses only
10-15 % of the roughly 68k-token budget a GPU holds; "LingBot-VA attention
profiling" report, conclusion and next steps: concatenating several episodes
(5-8 per GPU) along the sequence axis in the collate step fills that budget.

Reading taken: episodes arrive in the sampler's order and are concatenated in
that order; a pack is closed when the next episode would push it past the
budget, and that episode opens the next pack (next-fit).  An episode longer
than the budget cannot be placed and is an error.
"""
from __future__ import annotations

from typing import List


def next_fit_packs(lengths, budget: int) -> List[List[int]]:
    """Episode indices of each pack, in order."""
    if budget < 1:
        raise ValueError("budget must be >= 1")
    packs: List[List[int]] = []
    used = 0
    for e, n in enumerate(list(lengths)):
        n = int(n)
        if n < 0 or n > budget:
            raise ValueError(f"episode {e} has {n} tokens; the budget is {budget}")
        if not packs or used + n > budget:
            packs.append([])
            used = 0
        packs[-1].append(e)
        used += n
    return packs
