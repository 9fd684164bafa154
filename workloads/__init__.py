"""Seeded synthetic inputs for packed segment-id attention.

This package only draws inputs: episode lengths, padded frame counts, per-token
segment ids given directly (long mixed-modality pack, scattered pack), episode token counts
of unpadded packs, the random q, k, v, dO values, the random predictions /
targets of the masked loss and the AdaLN activations and modulation tables.  It holds none of the attention arithmetic and none
of the seq-id, packing or block-mask construction, so both the CPU oracle and
the HIP path can be fed from it without sharing any of the method's code.
"""
from .packs import (  # noqa: F401
    PackSpec,
    CONFIG_NAMES,
    config,
    bucketed_sweep,
    round_to_bf16,
    make_values,
    make_sweep_values,
    make_loss_values,
    make_adaln_values,
    UNPADDED_BUDGET,
    episode_stream,
    unpadded_pack,
    scattered_pack,
)
