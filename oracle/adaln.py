"""Oracle: AdaLN (LayerNorm followed by a per-segment modulation) on a packed
sequence, forward and backward (TEST INFRASTRUCTURE -- see ``oracle/__init__.py``).

AdaptiveLoad summary, section 2B (fused LayerNorm-Modulate kernel): each row is
normalised with its own mean and variance over the feature dimension D, and
the result is modulated (scaled and shifted) by conditioning-dependent
vectors; the backward reduces the modulation gradients over the sequence
dimension N.

Readings taken (the page gives no formula):
  * LayerNorm without its own affine parameters, biased variance, epsilon
    inside the square root:  xhat = (x - mean) / sqrt(var + eps);
  * modulation in the DiT form  y = xhat * (1 + scale) + shift;
  * on a packed sequence every episode (segment) has its own conditioning, so
    scale and shift are [S, D] tables and row i uses the row of its segment;
    segment s covers rows offsets[s] .. offsets[s+1]-1 (episodes are stored
    back to back); rows before offsets[0] or from offsets[S] on belong to no
    segment; offsets are first clamped into [0, N] and made non-decreasing
    (running maximum), so segments never overlap;
  * a row is valid iff its seq id is >= 0 and it lies in a segment; invalid
    rows (frame padding) give y = 0, mean = rstd = 0, dx = 0 and add nothing
    to the modulation gradients.
Backward for upstream gradient dy (chain rule of the forward):
    g = dy * (1 + scale[s]),
    dx = rstd * (g - mean_D(g) - xhat * mean_D(g * xhat)),
    d_scale[s] = sum over valid rows of segment s of dy * xhat,
    d_shift[s] = sum over valid rows of segment s of dy.
"""
from __future__ import annotations

import numpy as np


def segment_of_rows(offsets, n: int) -> np.ndarray:
    """Segment index of each of n rows (-1 outside every segment)."""
    seg = np.full(int(n), -1, dtype=np.int64)
    off = []
    for o in list(offsets):
        o = min(max(int(o), 0), int(n))
        off.append(max(o, off[-1]) if off else o)
    for s in range(len(off) - 1):
        for i in range(off[s], off[s + 1]):
            seg[i] = s
    return seg


def forward(x, seq_id, offsets, shift, scale, eps: float = 1e-6):
    """Return (y, mean, rstd) in fp64; y is [N, D], mean and rstd are [N]."""
    x = np.asarray(x, dtype=np.float64)
    shift = np.asarray(shift, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    n, d = x.shape
    seg = segment_of_rows(offsets, n)
    y = np.zeros((n, d))
    mean = np.zeros(n)
    rstd = np.zeros(n)
    for i in range(n):
        s = seg[i]
        if s < 0 or seq_id[i] < 0:
            continue
        mu = x[i].mean()
        var = ((x[i] - mu) ** 2).mean()
        r = 1.0 / np.sqrt(var + eps)
        xhat = (x[i] - mu) * r
        y[i] = xhat * (1.0 + scale[s]) + shift[s]
        mean[i], rstd[i] = mu, r
    return y, mean, rstd


def backward(x, dy, seq_id, offsets, scale, eps: float = 1e-6):
    """Return (dx, d_shift, d_scale) in fp64 for the forward above."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    n, d = x.shape
    n_seg = scale.shape[0]
    seg = segment_of_rows(offsets, n)
    dx = np.zeros((n, d))
    d_shift = np.zeros((n_seg, d))
    d_scale = np.zeros((n_seg, d))
    for i in range(n):
        s = seg[i]
        if s < 0 or seq_id[i] < 0:
            continue
        mu = x[i].mean()
        r = 1.0 / np.sqrt(((x[i] - mu) ** 2).mean() + eps)
        xhat = (x[i] - mu) * r
        g = dy[i] * (1.0 + scale[s])
        dx[i] = r * (g - g.mean() - xhat * (g * xhat).mean())
        d_scale[s] += dy[i] * xhat
        d_shift[s] += dy[i]
    return dx, d_shift, d_scale
