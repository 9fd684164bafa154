"""Checks of the seeded synthetic workloads (shapes, length mix, rounding)."""
import numpy as np
import torch

import workloads as wl


def test_config_shapes():
    assert wl.config(1).nq == 96 and wl.config(1).heads == 1 and wl.config(1).head_dim == 64
    assert wl.config(2).nq == 15360
    s3 = wl.config(3)
    assert s3.nq == 36864 and s3.nkv == 36864 and (s3.heads, s3.head_dim) == (24, 128)
    # padded to the next multiple of 8 frames above the longest episode
    assert s3.frames_padded == 288 == (int(s3.valid_frames.max()) + 7) // 8 * 8


def test_bucketed_sweep_statistics():
    sweep = wl.bucketed_sweep()
    assert len(sweep) == 40
    frames = np.concatenate([s.valid_frames for s in sweep])
    assert len(frames) == 160 and frames.min() >= 103 and frames.max() <= 362
    padded = [s.frames_padded for s in sweep]
    assert all(p % 8 == 0 and p >= s.valid_frames.max() for p, s in zip(padded, sweep))
    waste = 1 - frames.sum() / sum(4 * p for p in padded)
    assert abs(waste - 0.02667) < 1e-4
    assert len(set(padded)) == 30
    assert sum(s.nq for s in sweep) == 1251328
    assert max(s.nq for s in sweep) == 47104 == wl.config(4).nq
    cross = wl.bucketed_sweep(cross=True)
    assert [c.valid_frames.tolist() for c in cross] == [s.valid_frames.tolist() for s in sweep]
    assert sum(c.nq for c in cross) == 234624 and cross[0].cross


def test_long_mixed_pack():
    s = wl.config(5)
    ids = s.segment_ids
    assert len(ids) == 64000
    lengths = np.bincount(ids[ids >= 0])
    videos = [int(x) for x in lengths if x > 256]
    assert videos == [9139, 4767, 10554, 18144, 5558, 4183]
    assert int((lengths == 256).sum()) == 45 and int((ids < 0).sum()) == 135
    # padding only at the end
    assert (ids[-135:] == -1).all() and (ids[:-135] >= 0).all()


def test_scattered_pack():
    """Same token count per segment as the frame-padded 4 x 288 pack, reordered in
    512-token pieces: the segments are no longer contiguous."""
    s = wl.scattered_pack()
    ids = s.segment_ids
    assert s.nq == s.nkv == 36864 and (s.heads, s.head_dim) == (24, 128)
    assert np.bincount(ids[ids >= 0]).tolist() == [3808, 5664, 9120, 7648]
    assert int((ids < 0).sum()) == 36864 - 26240
    runs = 1 + int((ids[1:] != ids[:-1]).sum())
    assert runs > 40                      # scattered: many runs instead of 4 + padding
    pieces = ids.reshape(72, 512)
    assert sorted(map(bytes, pieces)) != [bytes(p) for p in pieces]  # reordered


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3e38, -1e-40], np.float32)])
    ours = wl.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_values_deterministic_and_bf16_exact():
    s = wl.config(2, heads=2)
    a = wl.make_values(s)
    b = wl.make_values(s)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
        assert np.array_equal(wl.round_to_bf16(x), x)
    assert abs(float(a[0].std()) - 0.5) < 0.01 and abs(float(a[3].std()) - 1.0) < 0.01
