"""Synthetic packs that stand in for the pages' workloads.

The pages train on FurnitureBench episodes of 103-362 latent frames, four per
GPU, each padded to a multiple of 8 frames (LingBot-VA packing report, sections
2.1 and 3.1), and discuss long mixed-modality sequences of 48k-64k tokens
(AdaptiveLoad summary, sections 1 and 4).  Neither dataset is available, so
every pack here is drawn from a seeded generator with the same shapes, length
mix and padding structure.

Nothing in this module computes attention, seq ids or block masks: a spec
carries the episode lengths (valid frames), the padded frame count and the
tokens per frame; the consumers build ids from them.  The long mixed-modality
pack has no frame structure, so its spec carries the per-token segment ids
directly.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "PackSpec",
    "CONFIG_NAMES",
    "config",
    "bucketed_sweep",
    "round_to_bf16",
    "make_values",
    "make_sweep_values",
    "make_loss_values",
    "make_adaln_values",
    "UNPADDED_BUDGET",
    "episode_stream",
    "unpadded_pack",
    "scattered_pack",
]


@dataclass
class PackSpec:
    """One packed attention problem.

    Frame-structured packs (``segment_ids is None``): episode ``b`` has
    ``valid_frames[b]`` real frames followed by padding up to
    ``frames_padded``; a frame holds ``q_tokens_per_frame`` query tokens and
    ``kv_tokens_per_frame`` key/value tokens (equal for self-attention).
    """

    name: str
    heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    seed: object  # anything np.random.default_rng accepts
    value_std: float = 1.0  # std of q, k, v; dO is always N(0, 1)
    valid_frames: Optional[np.ndarray] = None
    frames_padded: int = 0
    q_tokens_per_frame: int = 0
    kv_tokens_per_frame: int = 0
    segment_ids: Optional[np.ndarray] = None  # given directly (no frames)
    token_lengths: Optional[np.ndarray] = None  # unpadded pack: tokens per episode
    n_tokens: int = 0  # unpadded pack: fixed id-buffer length (the token budget)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def cross(self) -> bool:
        return (self.segment_ids is None and self.token_lengths is None
                and self.q_tokens_per_frame != self.kv_tokens_per_frame)

    @property
    def n_episodes(self) -> int:
        return 0 if self.valid_frames is None else int(len(self.valid_frames))

    @property
    def nq(self) -> int:
        if self.token_lengths is not None:
            return int(self.n_tokens)
        if self.segment_ids is not None:
            return int(len(self.segment_ids))
        return self.n_episodes * self.frames_padded * self.q_tokens_per_frame

    @property
    def nkv(self) -> int:
        if self.token_lengths is not None:
            return int(self.n_tokens)
        if self.segment_ids is not None:
            return int(len(self.segment_ids))
        return self.n_episodes * self.frames_padded * self.kv_tokens_per_frame

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out.

    Input preparation only: both sides of a parity test receive the same
    bf16-exact values.  NaN/Inf never occur in these generators.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def make_values(spec: PackSpec):
    """Draw q, k, v, dO as float32 arrays ``[n, heads, head_dim]``.

    Order of draws: q, k, v, dO from ``np.random.default_rng(spec.seed)``;
    q/k/v scaled by ``value_std``; bf16 specs are rounded to bf16 (RNE).
    """
    rng = np.random.default_rng(spec.seed)
    h, d = spec.heads, spec.head_dim
    out = []
    for n, std in ((spec.nq, spec.value_std), (spec.nkv, spec.value_std),
                   (spec.nkv, spec.value_std), (spec.nq, 1.0)):
        a = rng.standard_normal((n, h, d), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        if spec.dtype == "bf16":
            a = round_to_bf16(a)
        out.append(a)
    return tuple(out)


def make_sweep_values(n_q: int, n_kv: int, heads: int, head_dim: int, seed=(4, 999),
                      value_std: float = 0.5):
    """One set of bf16-exact values (float32 arrays ``[n, heads, head_dim]``) large
    enough for every batch of a sweep: a batch of nq query / nkv key tokens uses
    the first nq rows of q and dO and the first nkv rows of k and v.  Draws as in
    ``make_values`` (q, k, v, dO from ``np.random.default_rng(seed)``; q, k, v
    scaled by ``value_std``; dO ~ N(0, 1)), so one draw serves all batches."""
    rng = np.random.default_rng(list(seed))
    out = []
    for n, std in ((n_q, value_std), (n_kv, value_std), (n_kv, value_std), (n_q, 1.0)):
        a = rng.standard_normal((int(n), int(heads), int(head_dim)), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        out.append(round_to_bf16(a))
    return tuple(out)


def make_loss_values(n: int, channels: int, dtype: str, seed):
    """Draw a prediction and its target as float32 arrays ``[n, channels]``.

    Both ~ N(0, 1) from ``np.random.default_rng(seed)`` (prediction first);
    bf16 is rounded to bf16 (RNE).  Stand-ins for the latent (video) and
    action regression outputs whose loss is masked to valid frames.
    """
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(2):
        a = rng.standard_normal((int(n), int(channels)), dtype=np.float32)
        out.append(round_to_bf16(a) if dtype == "bf16" else a)
    return tuple(out)


def make_adaln_values(n: int, dim: int, n_seg: int, dtype: str, seed, mod_std: float = 0.5):
    """Draw AdaLN inputs: x [n, dim] with a random scale in [0.5, 2) and offset
    ~ N(0, 1) per row (so the normalisation has work to do), dy [n, dim] ~ N(0, 1),
    and the per-segment modulation tables shift, scale [n_seg, dim] ~ N(0, mod_std)
    (always fp32).  x and dy are rounded to bf16 for bf16.  Draw order: x, the
    row scales, the row offsets, dy, shift, scale."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((int(n), int(dim)), dtype=np.float32)
    x *= rng.uniform(0.5, 2.0, (int(n), 1)).astype(np.float32)
    x += rng.standard_normal((int(n), 1), dtype=np.float32)
    dy = rng.standard_normal((int(n), int(dim)), dtype=np.float32)
    shift = (mod_std * rng.standard_normal((int(n_seg), int(dim)))).astype(np.float32)
    scale = (mod_std * rng.standard_normal((int(n_seg), int(dim)))).astype(np.float32)
    if dtype == "bf16":
        x, dy = round_to_bf16(x), round_to_bf16(dy)
    return x, dy, shift, scale


def _pad_multiple(f: int, m: int = 8) -> int:
    return (int(f) + m - 1) // m * m


def _long_mixed_ids(total: int = 64000, seed: int = 0) -> np.ndarray:
    """Segment ids of one long mixed-modality sequence.

    While at least one image (256 tokens) still fits: with probability 0.3 a
    video of 4096..20480 tokens (an image instead if it would overflow), else
    a 256-token image.  The remainder past the last segment is padding (-1).
    """
    rng = np.random.default_rng(seed)
    lengths: List[int] = []
    rem = total
    while rem >= 256:
        if rng.random() < 0.3:
            n = int(rng.integers(4096, 20481))
            if n > rem:
                n = 256
        else:
            n = 256
        lengths.append(n)
        rem -= n
    ids = np.full(total, -1, dtype=np.int32)
    pos = 0
    for e, n in enumerate(lengths):
        ids[pos:pos + n] = e
        pos += n
    return ids


def bucketed_sweep(cross: bool = False, seed: int = 0, n_episodes: int = 160,
                   batch: int = 4, pool: int = 200) -> List[PackSpec]:
    """Length-bucketed batches: ``n_episodes`` lengths ~ U[103, 362] frames.

    Follows the bucket sampler the packing report describes (section 2.1): a
    seeded shuffle, pools of ``pool`` episodes sorted by length (stable), cut
    into batches of ``batch``, batch order shuffled; each batch padded to the
    next multiple of 8 frames.  One shard (no rank split).  Self-attention has
    32 video tokens per frame; the cross variant has 6 action tokens per frame
    querying the 32 video tokens.
    """
    frames = np.random.default_rng(seed).integers(103, 363, n_episodes)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_episodes)
    batches = []
    for p0 in range(0, n_episodes, pool):
        chunk = perm[p0:p0 + pool]
        chunk = chunk[np.argsort(frames[chunk], kind="stable")]
        for b0 in range(0, len(chunk) - batch + 1, batch):
            batches.append(chunk[b0:b0 + batch])
    order = rng.permutation(len(batches))
    specs = []
    for i, bi in enumerate(order):
        eps = batches[bi]
        vf = frames[eps].astype(np.int32)
        specs.append(PackSpec(
            name=f"bucketed{'-cross' if cross else ''}-b{i:02d}",
            heads=24, head_dim=128, dtype="bf16", seed=[4, int(i)],
            value_std=0.5, valid_frames=vf, frames_padded=_pad_multiple(vf.max()),
            q_tokens_per_frame=6 if cross else 32, kv_tokens_per_frame=32,
            notes="length-bucketed batch of 4"))
    return specs


UNPADDED_BUDGET = 68_000  # tokens per GPU ("about 68k", LingBot-VA packing report, section 1)


def episode_stream(seed: int = 0, n_episodes: int = 160, tokens_per_frame: int = 32):
    """Token counts of a stream of episodes in arrival order: frames ~ U[103, 362]
    (the same draw as ``bucketed_sweep``) times ``tokens_per_frame``, no padding."""
    frames = np.random.default_rng(seed).integers(103, 363, n_episodes)
    return (frames * int(tokens_per_frame)).astype(np.int32)


def unpadded_pack(token_lengths, name: str = "unpadded-68k", budget: int = UNPADDED_BUDGET,
                  heads: int = 24, head_dim: int = 128, seed=6) -> PackSpec:
    """An unpadded pack of the given episodes (consumers build the ids from the
    lengths) in an id buffer of ``budget`` tokens; values as the other bf16 packs."""
    return PackSpec(name, heads=heads, head_dim=head_dim, dtype="bf16", seed=seed,
                    value_std=0.5, token_lengths=np.asarray(token_lengths, np.int32),
                    n_tokens=int(budget), notes="episodes back to back, no frame padding")


def scattered_pack(chunk: int = 512, seed: int = 0) -> PackSpec:
    """The 4 x 288-frame pack's token counts in scattered order (segment ids given).

    Four segments of 119, 177, 285 and 239 frames x 32 tokens laid end to end,
    then padding (-1) up to the same 36,864 tokens; the sequence is cut into
    ``chunk``-token pieces that a seeded permutation reorders.  Every segment
    keeps its token count, so the allowed pairs (and the useful work) equal
    those of the frame-padded pack, while every query tile's key list is
    spread over the whole sequence (ids need not be sorted or contiguous).
    """
    lengths = np.array([119, 177, 285, 239], np.int64) * 32
    total = 4 * 288 * 32
    ids = np.full(total, -1, dtype=np.int32)
    ids[:lengths.sum()] = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
    pieces = ids.reshape(total // chunk, chunk)
    order = np.random.default_rng(seed).permutation(len(pieces))
    return PackSpec(f"var-4x288-scattered-{chunk}", heads=24, head_dim=128, dtype="bf16",
                    seed=7, value_std=0.5, segment_ids=np.ascontiguousarray(pieces[order]).ravel(),
                    notes=f"4x288 token counts, {chunk}-token pieces permuted")


CONFIG_NAMES = ("tiny-f32", "equal-4x120", "var-4x288", "bucketed", "long-64k")


def config(i: int, heads: Optional[int] = None) -> PackSpec:
    """The five workloads (1-based).  ``heads`` overrides the head count.

    1 tiny fp32 pack: valid frames 3/5/2 padded to 8, 4 tokens/frame, 1x64.
    2 four equal 120-frame episodes, 32 tokens/frame, 24x128 bf16.
    3 four episodes of 119/177/285/239 frames padded to 288 (the packing
      report's variable-length check, section 3.1), 24x128 bf16.
    4 the largest batch of the length-bucketed sweep (the whole sweep is
      ``bucketed_sweep``).
    5 one 64,000-token mixed image/video sequence, 24x128 bf16.
    """
    if i == 1:
        s = PackSpec("tiny-f32", heads=1, head_dim=64, dtype="f32", seed=1,
                     value_std=1.0, valid_frames=np.array([3, 5, 2], np.int32),
                     frames_padded=8, q_tokens_per_frame=4, kv_tokens_per_frame=4)
    elif i == 2:
        s = PackSpec("equal-4x120", heads=24, head_dim=128, dtype="bf16", seed=2,
                     value_std=0.5, valid_frames=np.array([120] * 4, np.int32),
                     frames_padded=120, q_tokens_per_frame=32, kv_tokens_per_frame=32)
    elif i == 3:
        s = PackSpec("var-4x288", heads=24, head_dim=128, dtype="bf16", seed=3,
                     value_std=0.5, valid_frames=np.array([119, 177, 285, 239], np.int32),
                     frames_padded=288, q_tokens_per_frame=32, kv_tokens_per_frame=32)
    elif i == 4:
        sweep = bucketed_sweep()
        s = max(sweep, key=lambda p: p.nq)
    elif i == 5:
        s = PackSpec("long-64k", heads=24, head_dim=128, dtype="bf16", seed=5,
                     value_std=0.5, segment_ids=_long_mixed_ids())
    else:
        raise ValueError(f"no workload {i}")
    if heads is not None:
        s.heads = int(heads)
    return s
