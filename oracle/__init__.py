"""CPU oracle for block-sparse attention prefill and the pooled attention map.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only the tests, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP library.

What it computes, each function citing the passage it follows:

* ``mask``    -- per-row threshold / TopK block selection on soft block scores
                 (model card of "SeerAttention-Llama-3.1-8B-AttnGates", method
                 summary; rebuttal "SeerAttention: Learning Intrinsic Sparse
                 Attention in Your LLMs", "Weakness 2 (Memory complexity)").
* ``attention`` -- causal attention restricted to the selected 64x64 blocks,
                 written as a plain masked softmax followed by P.V (the
                 rebuttal's "Weakness 5 (Pseudo code of Inference Kernel)"
                 computes the same thing block by block).
* ``pooled``  -- dense causal attention plus the 2D max-pooled probability map
                 (reproducibility summary of "SeerAttention: Self-distilled
                 Attention Gating for Efficient Long-context Prefilling",
                 Pseudocode row, Figure 8).
* ``gate``    -- the AttnGate's soft block scores: pooled Q and K, linear layers,
                 block RoPE and a causal softmax (rebuttal "SeerAttention:
                 Learning Intrinsic Sparse Attention in Your LLMs", Weakness 3
                 and the pooling and RoPE answers); and the per-token gate of
                 decoding, without query pooling (abstract of "SeerAttention-R").
* ``decode``  -- block-sparse attention of one new token over a KV cache and its
                 block selection with a token budget (abstract of "SeerAttention-R:
                 Sparse Attention Adaptation for Long Reasoning").
* ``target``  -- the row-normalised map used as the gate's ground truth and the
                 MSE against gate scores (rebuttal "SeerAttention: Learning
                 Intrinsic Sparse Attention in Your LLMs", "Question 2:
                 (Row-Normalization of Max-Pooled Attention Map)" and "Question
                 2 (Currently use MSE loss, how about e2e LM loss?)").

Everything is evaluated in float64 on the exact input values (bf16 inputs are
widened exactly).  The pins that tie these definitions to something other than
themselves live in ``tests/test_oracle_*.py``.
"""

from .mask import (MODE_THRESHOLD, MODE_TOPK, forced_blocks, topk_count, select_row,
                   build_mask_ref, mask_rows_ref, row_need, build_mask_need_ref,
                   validate_row_ref, validate_lists_ref, LIST_BAD_COUNT, LIST_BAD_ENTRY,
                   LIST_REPEAT, LIST_UNSORTED, LIST_CAPACITY)
from .attention import (BLOCK, block_probs, allowed_blocks, sparse_attention_ref,
                        sparse_attention_blocks_ref)
from .pooled import pooled_map_ref, pooled_map_blocks_ref
from .target import pooled_target_ref
from .gate import (pool_qk, block_rope, gate_qk_ref, gate_scores_ref, rope_at,
                   decode_gate_scores_ref)
from .decode import decode_blocks, select_decode_row, build_mask_decode_ref, sparse_decode_ref

__all__ = [
    "MODE_THRESHOLD", "MODE_TOPK", "BLOCK", "forced_blocks", "topk_count", "select_row",
    "build_mask_ref", "mask_rows_ref", "row_need", "build_mask_need_ref", "validate_row_ref",
    "validate_lists_ref", "LIST_BAD_COUNT", "LIST_BAD_ENTRY", "LIST_REPEAT", "LIST_UNSORTED",
    "LIST_CAPACITY", "block_probs", "allowed_blocks",
    "sparse_attention_ref", "sparse_attention_blocks_ref", "pooled_map_ref",
    "pooled_map_blocks_ref", "pooled_target_ref", "pool_qk", "block_rope", "gate_qk_ref",
    "gate_scores_ref", "rope_at", "decode_gate_scores_ref", "decode_blocks", "select_decode_row", "build_mask_decode_ref",
    "sparse_decode_ref",
]
