"""Oracle: frame-valid masked squared-error loss (TEST INFRASTRUCTURE).

"LingBot-VA packing" report, section 2.1 (compute_loss) and "Furniture packing,
variable length" report (implementation part): with packed, padded batches the
latent and action losses are averaged over the valid frames only, padding
frames excluded (frame_valid = arange(F) < valid_frames[:, None]).

Reading taken: the per-element loss is the squared error of a prediction
against its target (the flow-matching regression the model is trained with);
a token is valid iff its seq id is >= 0 (padding frames carry -1); the loss is
the mean over valid tokens and channels:
    L = sum_{i valid} sum_c (pred[i,c] - target[i,c])^2 / (n_valid * C),
and L = 0 when no token is valid.  Its gradient w.r.t. pred is
2 (pred - target) / (n_valid * C) on valid rows and 0 on padding rows.
Equal tokens per frame make the token mean equal to the mean over valid frames.
"""
from __future__ import annotations

import numpy as np


def masked_mse(pred, target, seq_ids, upstream: float = 1.0):
    """Return (loss, n_valid, dpred) in fp64; dpred = upstream * dL/dpred."""
    pred = np.asarray(pred, dtype=np.float64)
    target = np.asarray(target, dtype=np.float64)
    ids = np.asarray(seq_ids)
    n, c = pred.shape
    total = 0.0
    n_valid = 0
    for i in range(n):
        if ids[i] >= 0:
            n_valid += 1
            diff = pred[i] - target[i]
            total += float(diff @ diff)
    dpred = np.zeros((n, c))
    if n_valid == 0:
        return 0.0, 0, dpred
    denom = n_valid * c
    for i in range(n):
        if ids[i] >= 0:
            dpred[i] = upstream * 2.0 * (pred[i] - target[i]) / denom
    return total / denom, n_valid, dpred
