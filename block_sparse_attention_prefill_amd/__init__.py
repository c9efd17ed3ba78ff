"""MI355X-native block-sparse attention prefill (SeerAttention hot path).

The computation lives in libseer.so (HIP kernels for gfx950 behind the C-ABI of
include/seer.h); this package only marshals torch tensors into that library.
"""

from .binding import (BLOCK, SEER_MASK_THRESHOLD, SEER_MASK_TOPK, SeerError, load,
                      attn_gate_decode_keys_workspace_size, attn_gate_mask_pass_workspace_size,
                      attn_gate_mask_workspace_size,
                      attn_gate_workspace_size, seer_attn_gate_decode_keys,
                      seer_attn_gate_decode_mask, seer_attn_gate_decode_scores,
                      seer_attn_gate_mask, seer_attn_gate_scores, seer_build_mask_decode, seer_sparse_decode,
                      sparse_decode_workspace_size,
                      pooled_attn_map_workspace_size, seer_build_mask, seer_pooled_attn_map,
                      seer_pooled_target_mse, seer_sparse_prefill, seer_sparse_prefill_block,
                      sparse_prefill_workspace_size, topk_budget, version,
                      seer_build_mask_need, seer_validate_lists, list_flags_status,
                      seer_sparse_prefill_noalloc,
                      SEER_LIST_BAD_COUNT, SEER_LIST_BAD_ENTRY, SEER_LIST_REPEAT,
                      SEER_LIST_UNSORTED, SEER_LIST_CAPACITY)

__all__ = [
    "BLOCK", "SEER_MASK_THRESHOLD", "SEER_MASK_TOPK", "SeerError", "load",
    "attn_gate_decode_keys_workspace_size", "attn_gate_mask_pass_workspace_size",
    "attn_gate_mask_workspace_size",
    "attn_gate_workspace_size", "seer_attn_gate_decode_keys", "seer_attn_gate_decode_mask",
    "seer_attn_gate_decode_scores",
    "seer_attn_gate_mask",
    "seer_attn_gate_scores", "seer_build_mask_decode", "seer_sparse_decode",
    "sparse_decode_workspace_size",
    "pooled_attn_map_workspace_size", "seer_build_mask", "seer_pooled_attn_map",
    "seer_pooled_target_mse", "seer_sparse_prefill", "seer_sparse_prefill_block",
    "sparse_prefill_workspace_size", "topk_budget", "version", "seer_build_mask_need",
    "seer_validate_lists", "list_flags_status", "seer_sparse_prefill_noalloc", "SEER_LIST_BAD_COUNT", "SEER_LIST_BAD_ENTRY",
    "SEER_LIST_REPEAT", "SEER_LIST_UNSORTED", "SEER_LIST_CAPACITY",
]
