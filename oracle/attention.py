"""Oracle: packed segment-id masked attention, forward and backward, fp64.

TEST INFRASTRUCTURE -- see ``oracle/__init__.py``.

What is computed (the plain definition; the GPU path reaches the same result
up to rounding):

* Allowed pairs ("Furniture packing, variable length" report, implementation
  part; "LingBot-VA attention profiling" report, next steps): query i sees key
  j iff ``q_id[i] == kv_id[j] >= 0``.  A negative id is padding, removed both
  as query and as key ("LingBot-VA packing" report, section 2.1).
* The packing report's verification (section 2.2) compares the packed run
  with each episode run on its own; so the oracle does exactly that: for each
  id ``e >= 0`` it gathers the queries and the keys carrying ``e`` and runs
  dense softmax attention on them alone, per head:
      S = scale * Q K^T,  LSE = log sum_j exp(S_ij),  P = exp(S - LSE),
      O = P V.
  Backward with upstream gradient dO (standard softmax-attention gradient):
      dP = dO V^T,  Delta_i = sum_j P_ij dP_ij,  dS = P * (dP - Delta),
      dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
* A query with no allowed key (padding, or an id no key carries) gets
  O = 0, LSE = -inf and dQ = 0; a key no query selects gets dK = dV = 0.  The
  packing report's section 3.1 table only requires no NaN in these rows; zero
  output and -inf LSE is the reading taken.

Inputs are upcast to fp64 (bf16 and fp32 values are exact in fp64).  Query
rows of a long segment are processed in chunks of at most ``row_chunk``:
rows are independent and dK, dV are sums over rows, so chunking is exact up to
fp64 summation order.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def _episode_ids(q_ids: np.ndarray) -> list:
    return sorted(set(int(e) for e in q_ids[q_ids >= 0].tolist()))


def _heads(h_total: int, heads: Optional[Iterable[int]]):
    return list(range(h_total)) if heads is None else [int(h) for h in heads]


def forward(q, k, v, q_ids, kv_ids, scale: float, heads=None, row_chunk: int = 4096):
    """Return ``(o [nq, H, d], lse [H, nq])`` in fp64.

    ``heads`` restricts the work to a subset of heads; the other heads are
    left as NaN so that a caller cannot mistake them for results.
    """
    q_ids = np.asarray(q_ids)
    kv_ids = np.asarray(kv_ids)
    nq, h_total, d = q.shape
    hs = _heads(h_total, heads)
    o = np.full((nq, h_total, d), np.nan)
    lse = np.full((h_total, nq), np.nan)
    o[:, hs, :] = 0.0
    lse[hs, :] = -np.inf
    for e in _episode_ids(q_ids):
        qi = np.flatnonzero(q_ids == e)
        kj = np.flatnonzero(kv_ids == e)
        if len(kj) == 0:
            continue
        for h in hs:
            K = k[kj, h, :].astype(np.float64)
            V = v[kj, h, :].astype(np.float64)
            for c0 in range(0, len(qi), row_chunk):
                rows = qi[c0:c0 + row_chunk]
                Q = q[rows, h, :].astype(np.float64)
                S = scale * (Q @ K.T)
                m = S.max(axis=1)
                L = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
                P = np.exp(S - L[:, None])
                o[rows, h, :] = P @ V
                lse[h, rows] = L
    return o, lse


def forward_backward(q, k, v, dout, q_ids, kv_ids, scale: float, heads=None,
                     row_chunk: int = 4096):
    """Forward and backward in one pass.

    Returns a dict with ``o``, ``lse``, ``delta`` (``[H, nq]``, the row sums
    of P*dP, 0 on rows with no allowed key), ``dq``, ``dk``, ``dv``, all fp64.
    Heads outside ``heads`` are NaN.
    """
    q_ids = np.asarray(q_ids)
    kv_ids = np.asarray(kv_ids)
    nq, h_total, d = q.shape
    nkv = k.shape[0]
    hs = _heads(h_total, heads)

    def blank(shape, fill):
        a = np.full(shape, np.nan)
        a[(slice(None), hs) if len(shape) == 3 else (hs,)] = fill
        return a

    o = blank((nq, h_total, d), 0.0)
    dq = blank((nq, h_total, d), 0.0)
    dk = blank((nkv, h_total, d), 0.0)
    dv = blank((nkv, h_total, d), 0.0)
    lse = blank((h_total, nq), -np.inf)
    delta = blank((h_total, nq), 0.0)
    for e in _episode_ids(q_ids):
        qi = np.flatnonzero(q_ids == e)
        kj = np.flatnonzero(kv_ids == e)
        if len(kj) == 0:
            continue
        for h in hs:
            K = k[kj, h, :].astype(np.float64)
            V = v[kj, h, :].astype(np.float64)
            dK = np.zeros_like(K)
            dV = np.zeros_like(V)
            for c0 in range(0, len(qi), row_chunk):
                rows = qi[c0:c0 + row_chunk]
                Q = q[rows, h, :].astype(np.float64)
                dO = dout[rows, h, :].astype(np.float64)
                S = scale * (Q @ K.T)
                m = S.max(axis=1)
                L = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
                P = np.exp(S - L[:, None])
                o[rows, h, :] = P @ V
                lse[h, rows] = L
                dP = dO @ V.T
                D = (P * dP).sum(axis=1)
                dS = P * (dP - D[:, None])
                dq[rows, h, :] = scale * (dS @ K)
                dK += scale * (dS.T @ Q)
                dV += P.T @ dO
                delta[h, rows] = D
            dk[kj, h, :] = dK
            dv[kj, h, :] = dV
    return dict(o=o, lse=lse, delta=delta, dq=dq, dk=dk, dv=dv)


def useful_pairs(q_ids, kv_ids) -> int:
    """Number of allowed (query, key) pairs per head: sum over ids of n_q * n_kv."""
    q_ids = np.asarray(q_ids)
    kv_ids = np.asarray(kv_ids)
    total = 0
    for e in _episode_ids(q_ids):
        total += int((q_ids == e).sum()) * int((kv_ids == e).sum())
    return total
