"""Shared helpers of the GPU parity tests (no method arithmetic here).

Tolerances (stated for every comparison of GPU values with the fp64 oracle):
  fp32 inputs: max|gpu - ref| <= 1e-5 * max|ref| per tensor;
  bf16 inputs: max|gpu - ref| <= 2e-2 * max|ref| and
               sum|gpu - ref| / sum|ref| <= 3e-3 per tensor,
  both over the rows that have at least one allowed pair; every other row must
  be exactly zero, and LSE must be -inf exactly where the oracle's is.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": dict(max_rel=1e-5, mean_rel=None), "bf16": dict(max_rel=2e-2, mean_rel=3e-3)}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """bf16-exact float32 host array -> device tensor of the working dtype."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(TORCH_DTYPE[dtype]).cuda()


def ids_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def row_has_pair(q_ids, kv_ids):
    """(query rows with an allowed key, key rows with an allowed query)."""
    q_ids, kv_ids = np.asarray(q_ids), np.asarray(kv_ids)
    kset = set(kv_ids[kv_ids >= 0].tolist())
    qset = set(q_ids[q_ids >= 0].tolist())
    q_ok = np.array([e >= 0 and e in kset for e in q_ids.tolist()], dtype=bool)
    k_ok = np.array([e >= 0 and e in qset for e in kv_ids.tolist()], dtype=bool)
    return q_ok, k_ok


def compare(name, got, ref, live_rows, dtype, heads=None):
    """Assert the stated tolerance on live rows and exact zeros elsewhere.

    ``got`` / ``ref`` are ``[n, H, d]`` fp64 arrays, ``live_rows`` a bool [n].
    Returns (max_rel, mean_rel) for reporting.
    """
    if heads is not None:
        got, ref = got[:, heads], ref[:, heads]
    dead = ~live_rows
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert (got[dead] == 0).all(), f"{name}: padding / unselected rows are not exactly zero"
    g, r = got[live_rows], ref[live_rows]
    if r.size == 0:
        return 0.0, 0.0
    err = np.abs(g - r)
    scale = np.abs(r).max()
    max_rel = float(err.max() / scale) if scale > 0 else float(err.max())
    mean_rel = float(err.sum() / max(np.abs(r).sum(), 1e-300))
    tol = TOL[dtype]
    assert max_rel <= tol["max_rel"], f"{name}: max|d|/max|ref| = {max_rel:.3e} > {tol['max_rel']}"
    if tol["mean_rel"] is not None:
        assert mean_rel <= tol["mean_rel"], f"{name}: sum|d|/sum|ref| = {mean_rel:.3e}"
    return max_rel, mean_rel


def compare_lse(got, ref, heads=None, atol=1e-3):
    """-inf pattern exact; finite entries within atol (natural-log units)."""
    if heads is not None:
        got, ref = got[heads], ref[heads]
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), "LSE -inf pattern differs"
    assert np.isfinite(got[~ninf]).all()
    if (~ninf).any():
        d = float(np.abs(got[~ninf] - ref[~ninf]).max())
        assert d <= atol, f"LSE max abs diff {d:.3e} > {atol}"


# ------------------------------------------------------------------ guard bands
GUARD = 4096  # canary elements on each side of a guarded buffer (>= 8 KB, keeps alignment)
_CANARY = {torch.bfloat16: (torch.int16, 0x7FA1), torch.float32: (torch.int32, 0x7FA00001),
           torch.int32: (torch.int32, -0x5A5A5A5B), torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """A device buffer that sits between two guard bands of a canary bit pattern
    (a NaN for floating types, one no kernel writes).  The interior starts as the
    same canary, so a row the kernel never writes is caught too (NaN, or the
    pattern itself for integer storage).  ``check()`` asserts both bands are
    untouched: a write past either end of the buffer fails it."""

    def __init__(self, shape, dtype, device="cuda"):
        n = 1
        for s in shape:
            n *= int(s)
        itype, bits = _CANARY[dtype]
        self.raw = torch.full((n + 2 * GUARD,), bits, dtype=itype, device=device)
        self.tensor = self.raw.view(dtype)[GUARD:GUARD + n].view(*shape)
        self.bits, self.n = bits, n

    def check(self, name="buffer"):
        lo, hi = self.raw[:GUARD], self.raw[GUARD + self.n:]
        assert bool((lo == self.bits).all()), f"{name}: write before the start of the buffer"
        assert bool((hi == self.bits).all()), f"{name}: write past the end of the buffer"
