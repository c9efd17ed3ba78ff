// Internal declarations shared by the HIP translation units of libseer.
// Not part of the public interface (that is include/seer.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace seer {

constexpr int kBlk = 64;  // tokens per query / KV block

// Vector types accepted by the gfx950 MFMA builtins.
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// int32 entries of the sparse prefill's work list (schedule output: one int4 per item).
size_t sparse_work_entries(int B, int Hq, int Hkv, int nqb);

// need may be null (no per-row untruncated counts).
hipError_t launch_build_mask(const float* scores, int B, int H, int nqb, int nkb, int mode,
                             float threshold, double density, int keep_sink, int32_t* idx,
                             int32_t* cnt, int32_t* need, int max_k, hipStream_t stream);

// List validation: rows = B*H*nB list rows of max_k entries; need and row_flags
// may be null; flags (one int) is cleared on the stream first.
hipError_t launch_validate_lists(const int32_t* idx, const int32_t* cnt, const int32_t* need,
                                 long long rows, int nrows_per_head, int max_k,
                                 int32_t* row_flags, int32_t* flags, hipStream_t stream);

// Decode rows: B*H rows of nkb scores; row (b, h) ranks the blocks holding
// kv_len[b] tokens (block tokens each).
hipError_t launch_build_mask_decode(const float* scores, const int32_t* kv_len, int B, int H,
                                    int nkb, int block, int mode, float threshold, int k_blocks,
                                    int keep_sink, int32_t* idx, int32_t* cnt, int max_k,
                                    hipStream_t stream);

// block: list block size in tokens, 64 or 128 (checked by the caller).
hipError_t launch_sparse_prefill(const void* q, const void* k, const void* v, int B, int Hq,
                                 int Hkv, int T, int D, float sm_scale, int block,
                                 const int32_t* idx, const int32_t* cnt, int max_k, int32_t* work,
                                 void* o, hipStream_t stream);

hipError_t launch_pooled_map(const void* q, const void* k, const void* v, int B, int Hq,
                             int Hkv, int T, int D, float sm_scale, void* o, float* amap,
                             float* rowmax_ws, hipStream_t stream);

hipError_t launch_pooled_target(const float* amap, const float* gate, int B, int H, int nqb,
                                float* target, float* row_sse, float* loss, hipStream_t stream);

// fp32 elements of the gate's workspace (projected Q~ and K~).
size_t attn_gate_workspace_floats(int B, int Hq, int Hkv, int nqb, int dg);

hipError_t launch_attn_gate(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                            const float* wq, const float* wk, int dg, float scale,
                            float rope_base, float* scores, float* ws, hipStream_t stream);

// Gate scores and block lists in one pass over the logits (nqb <= 4096, checked
// by the caller).  scores may be null: the logits then live in ws from the
// first 64-float boundary past attn_gate_workspace_floats(), pass_rows rows of
// nqb floats per head (B*Hq*pass_rows*nqb floats), and the rows are produced
// and selected in passes of pass_rows query blocks; pass_rows is nqb (one pass)
// or a multiple of 64 below it.  Ignored when scores is given.
hipError_t launch_attn_gate_mask(const void* q, const void* k, int B, int Hq, int Hkv, int T,
                                 int D, const float* wq, const float* wk, int dg, float scale,
                                 float rope_base, int mode, float threshold, double density,
                                 int keep_sink, int32_t* idx, int32_t* cnt, int max_k,
                                 float* scores, float* ws, int pass_rows, hipStream_t stream);

// Per-token decode gate (block 64 or 128, nKB = ceil(Tmax / block) <= 4096 and
// B * max(Hq, Hkv) * nKB < 2^31, checked by the caller).  Keys: kt [B,Hkv,nKB,Dg]
// for every block, or only each sequence's last block.  Scores from kt.
size_t attn_gate_decode_keys_workspace_floats(int B, int Hkv, int nkb, int D);
hipError_t launch_attn_gate_decode_keys(const void* k, const int32_t* kv_len, int B, int Hkv,
                                        int Tmax, int D, const float* wk, int dg,
                                        float rope_base, int block, int only_last,
                                        float* kt, float* ws, hipStream_t stream);
hipError_t launch_attn_gate_decode_scores(const void* q, const float* kt, const int32_t* kv_len,
                                          int B, int Hq, int Hkv, int Tmax, int D,
                                          const float* wq, int dg, float scale, float rope_base,
                                          int block, float* scores, hipStream_t stream);
// Decode gate scores straight into decode block lists (nKB <= 4096; the same
// argument rules as launch_build_mask_decode); scores may be null.
hipError_t launch_attn_gate_decode_mask(const void* q, const float* kt, const int32_t* kv_len,
                                        int B, int Hq, int Hkv, int Tmax, int D, const float* wq,
                                        int dg, float scale, float rope_base, int block,
                                        int mode, float threshold, int k_blocks, int keep_sink,
                                        int32_t* idx, int32_t* cnt, int max_k, float* scores,
                                        hipStream_t stream);

// Decode: workspace bytes and grid size of launch_sparse_decode (list_heads is
// Hq or Hkv; the caller checks the arguments).
size_t sparse_decode_workspace_bytes(int B, int Hq, int Hkv, int Tmax, int D, int list_heads,
                                     int max_k, int block);
long long sparse_decode_grid(int B, int Hq, int Hkv, int Tmax, int D, int list_heads, int max_k,
                             int block);
hipError_t launch_sparse_decode(const void* q, const void* k, const void* v,
                                const int32_t* kv_len, int B, int Hq, int Hkv, int Tmax, int D,
                                float sm_scale, int block, const int32_t* kv_idx,
                                const int32_t* kv_cnt, int list_heads, int max_k, void* o,
                                void* ws, hipStream_t stream);

}  // namespace seer
