"""Oracle: block sparsity of the same-seq-id mask.

TEST INFRASTRUCTURE -- see ``oracle/__init__.py``.

"LingBot-VA packing" report, section 1 and 2.2: the packed sequence is masked
by a block mask built from the seq ids, so whole blocks with no allowed pair
are skipped.  Pair predicate ("Furniture packing, variable length" report,
implementation part; "LingBot-VA attention profiling" report, next steps):
query i may attend key j iff ``q_id[i] == kv_id[j]`` and the id is not
negative -- a negative id is padding and is removed as query and as key.

For tile sizes ``bq x bkv`` the query axis is cut into ``ceil(nq/bq)`` tiles
and the key axis into ``ceil(nkv/bkv)`` tiles (the last ones may be short).
Class of a tile pair: 0 (empty) if it holds no allowed pair, 2 (full) if all
``bq*bkv`` positions are allowed pairs, 1 (partial) otherwise.  A short tail
tile is therefore never full.
"""
from __future__ import annotations

import numpy as np

EMPTY, PARTIAL, FULL = 0, 1, 2


def _tile_id_histogram(ids: np.ndarray, block: int, n_tiles: int, id_index: dict) -> np.ndarray:
    """Count, per tile, the tokens carrying each non-negative id."""
    h = np.zeros((n_tiles, max(len(id_index), 1)), dtype=np.float64)
    for pos, e in enumerate(ids.tolist()):
        if e >= 0:
            h[pos // block, id_index[e]] += 1.0
    return h


def tile_pair_counts(q_ids, kv_ids, bq: int, bkv: int) -> np.ndarray:
    """Number of allowed (query, key) pairs in every tile pair, int64.

    Allowed pairs with id ``e`` in tile pair (I, J) number ``cq[I, e] * ck[J, e]``
    where ``cq``/``ck`` count id ``e`` in the query/key tile; summing over ``e``
    is a product of the two histograms (exact: every count is far below 2**53).
    """
    q_ids = np.asarray(q_ids, dtype=np.int64)
    kv_ids = np.asarray(kv_ids, dtype=np.int64)
    nqt = -(-len(q_ids) // bq)
    nkt = -(-len(kv_ids) // bkv)
    uniq = sorted(set(q_ids[q_ids >= 0].tolist()) | set(kv_ids[kv_ids >= 0].tolist()))
    index = {e: c for c, e in enumerate(uniq)}
    cq = _tile_id_histogram(q_ids, bq, nqt, index)
    ck = _tile_id_histogram(kv_ids, bkv, nkt, index)
    return np.rint(cq @ ck.T).astype(np.int64)


def tile_classes(q_ids, kv_ids, bq: int, bkv: int) -> np.ndarray:
    """uint8 ``[nq_tiles, nkv_tiles]``: 0 empty, 1 partial, 2 full."""
    cnt = tile_pair_counts(q_ids, kv_ids, bq, bkv)
    cls = np.full(cnt.shape, PARTIAL, dtype=np.uint8)
    cls[cnt == 0] = EMPTY
    cls[cnt == bq * bkv] = FULL
    return cls


def csr_lists(cls: np.ndarray):
    """Non-empty tiles as two CSR structures, each list ascending.

    Returns ``(q_ptr, q_cols, kv_ptr, kv_rows)``: for query tile I the key
    tiles ``q_cols[q_ptr[I]:q_ptr[I+1]]``, and for key tile J the query tiles
    ``kv_rows[kv_ptr[J]:kv_ptr[J+1]]``.
    """
    nqt, nkt = cls.shape
    nz = cls != EMPTY
    rows, cols = np.nonzero(nz)          # row-major: ascending column within a row
    q_ptr = np.concatenate([[0], np.cumsum(nz.sum(axis=1))])
    cols_t, rows_t = np.nonzero(nz.T)    # column-major: ascending row within a column
    kv_ptr = np.concatenate([[0], np.cumsum(nz.sum(axis=0))])
    as32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
    return as32(q_ptr), as32(cols), as32(kv_ptr), as32(rows_t)


def class_totals(cls: np.ndarray):
    """(empty, partial, full) tile-pair counts."""
    return (int((cls == EMPTY).sum()), int((cls == PARTIAL).sum()), int((cls == FULL).sum()))


def longest_first_order(cls: np.ndarray, axis: int = 0) -> np.ndarray:
    """Tiles of one axis by decreasing number of non-empty partners, ties by
    ascending index (``axis`` 0: query tiles, 1: key tiles)."""
    lens = (cls != EMPTY).sum(axis=1 - axis)
    return np.asarray(sorted(range(len(lens)), key=lambda t: (-int(lens[t]), t)), dtype=np.int32)


def pair_lists(cls: np.ndarray, q_order: np.ndarray):
    """The walk of each pair of query tiles (positions 2w and 2w + 1 of the
    query order): every key tile that either tile has an allowed pair with,
    ascending, encoded ``kt | class(first) << 16 | class(second) << 24`` (class
    0 outside a tile's list and for a missing second tile).

    Returns ``(room, lists)``: ``room`` is the exclusive prefix sum over pairs of
    the two tiles' list lengths (``npairs + 1`` entries), ``lists`` one int32
    array per pair."""
    nqt, nkt = cls.shape
    lens = (cls != EMPTY).sum(axis=1)
    room, lists = [0], []
    for w in range((nqt + 1) // 2):
        a = int(q_order[2 * w])
        b = int(q_order[2 * w + 1]) if 2 * w + 1 < nqt else -1
        ra = cls[a].astype(np.int64)
        rb = cls[b].astype(np.int64) if b >= 0 else np.zeros(nkt, np.int64)
        cols = np.flatnonzero((ra != EMPTY) | (rb != EMPTY))  # ascending
        lists.append((cols | (ra[cols] << 16) | (rb[cols] << 24)).astype(np.int32))
        room.append(room[-1] + int(lens[a]) + (int(lens[b]) if b >= 0 else 0))
    return np.asarray(room, dtype=np.int32), lists
