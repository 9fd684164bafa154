"""GPU parity of the seq-id helper and the block-mask builder (bit-exact)."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import blockmask as obm
from oracle import seqids as osid
from tests._helpers import ids_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import packed_variable_length_amd as pa_mod
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return pa_mod


def _gpu_ids(pa, spec, tokens_per_frame):
    vf = ids_dev(spec.valid_frames)
    return pa.seq_ids_from_valid_frames(vf, spec.frames_padded, tokens_per_frame)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_seq_ids_match_oracle(pa, cfg):
    s = wl.config(cfg)
    got = _gpu_ids(pa, s, s.q_tokens_per_frame).cpu().numpy()
    want = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    assert np.array_equal(got, want)


def test_seq_ids_edge_cases(pa):
    for vf, fp, t in (([5, -2, 0, 3], 3, 2), ([0], 1, 1), ([7] * 9, 7, 5), ([1, 2], 4, 33)):
        got = pa.seq_ids_from_valid_frames(ids_dev(np.array(vf)), fp, t).cpu().numpy()
        assert np.array_equal(got, osid.seq_ids_from_valid_frames(vf, fp, t)), (vf, fp, t)


def _check_mask(pa, qid, kid, bq, bkv):
    m = pa.build_block_mask(ids_dev(qid), ids_dev(kid), bq, bkv)
    cls = m.tile_class().cpu().numpy()
    want = obm.tile_classes(qid, kid, bq, bkv)
    assert cls.shape == want.shape
    assert np.array_equal(cls, want), f"class matrix differs at {np.argwhere(cls != want)[:5]}"
    q_ptr, q_cols, kv_ptr, kv_rows = (t.cpu().numpy() for t in m.csr())
    wq_ptr, wq_cols, wkv_ptr, wkv_rows = obm.csr_lists(want)
    assert np.array_equal(q_ptr, wq_ptr) and np.array_equal(q_cols, wq_cols)
    assert np.array_equal(kv_ptr, wkv_ptr) and np.array_equal(kv_rows, wkv_rows)
    # longest-first orders (ties ascending: unique) and the pair walks
    q_order, kv_order = (t.cpu().numpy() for t in m.orders())
    assert np.array_equal(q_order, obm.longest_first_order(want, 0))
    assert np.array_equal(kv_order, obm.longest_first_order(want, 1))
    _check_pairs(m, want, q_order)
    return cls


def _check_pairs(m, want, q_order):
    off, ln, ent = (t.cpu().numpy() for t in m.pairs())
    room, lists = obm.pair_lists(want, q_order)
    assert np.array_equal(off, room)
    assert np.array_equal(ln, [len(x) for x in lists])
    for w, x in enumerate(lists):
        assert np.array_equal(ent[off[w]:off[w] + ln[w]], x), f"pair {w}"


def test_mask_closed_form_totals(pa):
    # hand-derived totals (tests/golden/tile_class_totals.txt)
    for cfg, bq, bkv, want in ((3, 128, 128, (71235, 410, 11299)), (3, 128, 64, (142587, 615, 22686)),
                               (2, 128, 128, (10800, 0, 3600)), (1, 32, 32, (6, 3, 0)),
                               (1, 64, 64, (2, 2, 0))):
        s = wl.config(cfg)
        ids = _gpu_ids(pa, s, s.q_tokens_per_frame)
        m = pa.build_block_mask(ids, ids, bq, bkv)
        assert obm.class_totals(m.tile_class().cpu().numpy()) == want, (cfg, bq, bkv)


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_mask_matches_oracle_configs(pa, cfg):
    s = wl.config(cfg)
    if s.segment_ids is not None:
        ids = s.segment_ids
    else:
        ids = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
    for bq, bkv in ((128, 128), (64, 128), (128, 32)):
        _check_mask(pa, ids, ids, bq, bkv)


def test_mask_cross_attention(pa):
    for s in wl.bucketed_sweep(cross=True)[:3]:
        qid = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.q_tokens_per_frame)
        kid = osid.seq_ids_from_valid_frames(s.valid_frames, s.frames_padded, s.kv_tokens_per_frame)
        _check_mask(pa, qid, kid, 128, 128)


@pytest.mark.parametrize("seed", range(5))
def test_mask_interleaved_and_ragged(pa, seed):
    # interleaved ids force the exact per-pair resolution path
    rng = np.random.default_rng(seed)
    nq, nkv = int(rng.integers(1, 3000)), int(rng.integers(1, 3000))
    nid = int(rng.integers(1, 40))
    qid = rng.integers(-3, nid, nq).astype(np.int32)
    kid = rng.integers(-3, nid, nkv).astype(np.int32)
    if seed == 3:
        qid = np.sort(qid)
    for bq, bkv in ((16, 16), (128, 128), (256, 64), (1024, 1024)):
        _check_mask(pa, qid, kid, bq, bkv)


def test_mask_large_ids(pa):
    # ids at and above 2^30 (and near the int32 maximum) classify like any other
    rng = np.random.default_rng(11)
    base = np.array([0, 5, (1 << 30) - 1, 1 << 30, (1 << 30) + 7, (1 << 31) - 2], np.int64)
    qid = np.repeat(base, 300).astype(np.int32)
    kid = np.repeat(base[::-1], 260).astype(np.int32)
    qid[rng.random(len(qid)) < 0.05] = -1
    for bq, bkv in ((128, 128), (64, 128), (256, 32)):
        _check_mask(pa, qid, kid, bq, bkv)
        _check_mask(pa, qid, qid, bq, bkv)


def test_mask_stress_1m_tokens(pa):
    # 1,048,576 tokens in 4096-token segments, with 2% padding tokens
    n = 1 << 20
    ids = (np.arange(n) // 4096).astype(np.int32)
    ids[np.random.default_rng(0).random(n) < 0.02] = -1
    m = pa.build_block_mask(ids_dev(ids), ids_dev(ids), 128, 128)
    cls = m.tile_class().cpu().numpy()
    want = obm.tile_classes(ids, ids, 128, 128)
    assert np.array_equal(cls, want)
    q_ptr, q_cols, kv_ptr, kv_rows = (t.cpu().numpy() for t in m.csr())
    wq_ptr, wq_cols, wkv_ptr, wkv_rows = obm.csr_lists(want)
    assert np.array_equal(q_ptr, wq_ptr) and np.array_equal(q_cols, wq_cols)
    assert np.array_equal(kv_ptr, wkv_ptr) and np.array_equal(kv_rows, wkv_rows)
    q_order = m.orders()[0].cpu().numpy()
    assert np.array_equal(q_order, obm.longest_first_order(want, 0))
    _check_pairs(m, want, q_order)
