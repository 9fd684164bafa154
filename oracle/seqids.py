"""Oracle: per-token seq ids from per-episode valid frame counts.

TEST INFRASTRUCTURE -- see ``oracle/__init__.py``.

"LingBot-VA packing" report, section 2.1: the mask builder takes the latent
and action seq-id grids of shape (B, F, H, W); a token whose frame index is at
or past ``valid_frames[b]`` gets -1, every other token of episode ``b`` gets
``b``; the collate step zero-pads every episode to the same padded frame count.
Token order (a reading, the pages give only the grid shape): episode-major,
then frame, then the frame's tokens.
"""
from __future__ import annotations

import numpy as np


def seq_ids_from_valid_frames(valid_frames, frames_padded: int, tokens_per_frame: int) -> np.ndarray:
    """Return int32 ids of length ``B * frames_padded * tokens_per_frame``.

    A ``valid_frames`` entry outside ``[0, frames_padded]`` is clamped into
    that range (negative means the whole episode is padding).
    """
    out = []
    for b, vf in enumerate(list(valid_frames)):
        vf = min(max(int(vf), 0), int(frames_padded))
        for f in range(int(frames_padded)):
            tag = b if f < vf else -1
            out.extend([tag] * int(tokens_per_frame))
    return np.asarray(out, dtype=np.int32)


def seq_ids_from_lengths(lengths, n_tokens: int) -> np.ndarray:
    """Seq ids of an unpadded pack: episodes concatenated back to back.

    "LingBot-VA attention profiling" report, next steps: the collate step
    concatenates K episodes along the sequence axis and gives every token its
    document id (here the episode's position in ``lengths``).  The id buffer
    has a fixed length ``n_tokens``: positions past the last episode are
    padding (-1); an episode that runs past ``n_tokens`` is cut there.  A
    negative length counts as 0.
    """
    out = np.full(int(n_tokens), -1, dtype=np.int32)
    pos = 0
    for e, n in enumerate(list(lengths)):
        for _ in range(max(int(n), 0)):
            if pos >= n_tokens:
                return out
            out[pos] = e
            pos += 1
    return out
