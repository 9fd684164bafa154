"""Packed segment-id masked attention for MI355X (gfx950).

The compute path is the HIP library ``libpackattn.so`` (C ABI in
``include/packattn.h``); :mod:`packed_variable_length_amd.packattn` is its thin
Python binding.  Importing this package fails if the library is not built.
"""
from .packattn import (  # noqa: F401
    PA_BF16,
    PA_F32,
    BlockMask,
    PackAttnError,
    adaln_bwd,
    adaln_bwd_workspace_bytes,
    adaln_fwd,
    attn_packed_bwd,
    attn_packed_bwd_dkdv,
    attn_packed_bwd_dq,
    attn_packed_bwd_noalloc,
    attn_packed_bwd_noalloc_max_bytes,
    attn_packed_bwd_preprocess,
    attn_packed_bwd_workspace_bytes,
    attn_packed_fwd,
    build_block_mask,
    build_block_mask_bytes,
    dual_constraint_batch,
    fit_step_cost,
    length_bucket_batches,
    masked_mse_bwd,
    masked_mse_fwd,
    masked_mse_fwd_bwd,
    masked_mse_workspace_bytes,
    pa_status_str,
    pa_test_set_handover_spin_limit,
    pa_handover_failures,
    plan_token_packs,
    seq_ids_from_lengths,
    seq_ids_from_valid_frames,
)
