// Host side of the C-ABI declared in include/seer.h: argument checks, workspace
// layout and kernel launches.  No allocation, no global mutable state.
#include "seer.h"

#include <math.h>
#include <limits.h>

#include <algorithm>
#include <mutex>

#include "seer_internal.h"

// Scratch of the no-allocation prefill entry point: the schedule's work list
// (16 bytes per 64-row item) for up to kNoAllocItems items.  Each GPU the
// library runs on holds one copy until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
namespace {
constexpr long long kNoAllocItems = 1 << 18;
}
static __device__ __align__(256) int32_t scratch[4 * kNoAllocItems];

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// In 64 bits: callers pass T before it is range-checked, and T + 63 overflows
// int for T near INT_MAX; the quotient always fits.
int nqb_of(int T) { return (int)(((long long)T + SEER_BLOCK - 1) / SEER_BLOCK); }

// Sizes must keep every flattened index inside int32 / size_t arithmetic the
// kernels use: item ids (B*H*nQB) are int, element offsets are size_t.
bool items_fit(long long B, long long H, long long nqb) {
  return B >= 0 && H >= 0 && nqb >= 0 && B * H * nqb <= (long long)INT_MAX;
}

int attention_args(const void* q, const void* k, const void* v, const void* o, int B, int Hq,
                   int Hkv, int T, int D, float sm_scale) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0) return SEER_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SEER_ERR_INVALID_ARG;
  if (!(isfinite(sm_scale) && sm_scale > 0.f)) return SEER_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SEER_ERR_UNSUPPORTED;
  if (!items_fit(B, Hq, nqb_of(T))) return SEER_ERR_UNSUPPORTED;
  if ((long long)B * T == 0) return SEER_OK;
  if (!q || !k || !v || !o) return SEER_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return SEER_ERR_INVALID_ARG;
  return SEER_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept for later calls.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SEER_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SEER_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SEER_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SEER_OK;
}

}  // namespace

extern "C" {

const char* seer_status_string(int status) {
  switch (status) {
    case SEER_OK: return "SEER_OK";
    case SEER_ERR_INVALID_ARG: return "SEER_ERR_INVALID_ARG";
    case SEER_ERR_UNSUPPORTED: return "SEER_ERR_UNSUPPORTED";
    case SEER_ERR_CAPACITY: return "SEER_ERR_CAPACITY";
    case SEER_ERR_WORKSPACE: return "SEER_ERR_WORKSPACE";
    case SEER_ERR_HIP: return "SEER_ERR_HIP";
    default: return "SEER_ERR_UNKNOWN";
  }
}

int seer_version(void) { return kVersion; }

int seer_topk_budget(int nQB, double density, int keep_sink) {
  if (nQB < 0 || !(density > 0.0 && density <= 1.0)) return -1;
  if (nQB == 0) return 0;
  const int i = nQB - 1;
  const int forced = (i == 0) ? 1 : (keep_sink ? 2 : 1);
  const double c = ceil(density * (double)(i + 1));
  int k = (int)c;
  if (k < forced) k = forced;
  if (k > i + 1) k = i + 1;
  return k;
}

}  // extern "C"

namespace {

int build_mask_impl(const float* scores, int B, int H, int nQB, int nKB, int mode,
                    float threshold, double density, int keep_sink, int32_t* kv_idx,
                    int32_t* kv_cnt, int32_t* kv_need, int max_k, void* stream) {
  if (B < 0 || H < 0 || nQB < 0 || nKB < nQB) return SEER_ERR_INVALID_ARG;
  if (nQB > SEER_MAX_QUERY_BLOCKS) return SEER_ERR_UNSUPPORTED;
  if (mode != SEER_MASK_TOPK && mode != SEER_MASK_THRESHOLD) return SEER_ERR_INVALID_ARG;
  if (!items_fit(B, H, nQB)) return SEER_ERR_UNSUPPORTED;
  if (mode == SEER_MASK_TOPK && !(density > 0.0 && density <= 1.0)) return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_THRESHOLD && !isfinite(threshold)) return SEER_ERR_INVALID_ARG;
  if (max_k < 1) return SEER_ERR_CAPACITY;
  if ((long long)B * H * nQB == 0) return SEER_OK;
  if (!scores || !kv_idx || !kv_cnt) return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_TOPK) {
    if (max_k < seer_topk_budget(nQB, density, keep_sink)) return SEER_ERR_CAPACITY;
  } else {
    const int forced = (keep_sink && nQB > 1) ? 2 : 1;
    if (max_k < forced) return SEER_ERR_CAPACITY;
  }
  const hipError_t err = seer::launch_build_mask(scores, B, H, nQB, nKB, mode, threshold,
                                                 density, keep_sink ? 1 : 0, kv_idx, kv_cnt,
                                                 kv_need, max_k, (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

}  // namespace

extern "C" {

int seer_build_mask(const float* scores, int B, int H, int nQB, int nKB, int mode,
                    float threshold, double density, int keep_sink, int32_t* kv_idx,
                    int32_t* kv_cnt, int max_k, void* stream) {
  return build_mask_impl(scores, B, H, nQB, nKB, mode, threshold, density, keep_sink, kv_idx,
                         kv_cnt, nullptr, max_k, stream);
}

int seer_build_mask_need(const float* scores, int B, int H, int nQB, int nKB, int mode,
                         float threshold, double density, int keep_sink, int32_t* kv_idx,
                         int32_t* kv_cnt, int32_t* kv_need, int max_k, void* stream) {
  if (!kv_need && (long long)B * H * nQB > 0) return SEER_ERR_INVALID_ARG;
  return build_mask_impl(scores, B, H, nQB, nKB, mode, threshold, density, keep_sink, kv_idx,
                         kv_cnt, kv_need, max_k, stream);
}

int seer_validate_lists(const int32_t* kv_idx, const int32_t* kv_cnt, const int32_t* kv_need,
                        int B, int H, int nB, int max_k, int32_t* row_flags, int32_t* flags,
                        void* stream) {
  if (B < 0 || H < 0 || nB < 0 || max_k < 1) return SEER_ERR_INVALID_ARG;
  if (!items_fit(B, H, nB)) return SEER_ERR_UNSUPPORTED;
  if (!flags) return SEER_ERR_INVALID_ARG;
  const long long rows = (long long)B * H * nB;
  if (rows > 0 && (!kv_idx || !kv_cnt)) return SEER_ERR_INVALID_ARG;
  const hipError_t err = seer::launch_validate_lists(kv_idx, kv_cnt, kv_need, rows, nB, max_k,
                                                     row_flags, flags, (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

int seer_list_flags_status(int flags) {
  if (flags & SEER_LIST_CAPACITY) return SEER_ERR_CAPACITY;
  if (flags & SEER_LIST_REPEAT) return SEER_ERR_INVALID_ARG;
  return SEER_OK;
}

size_t seer_sparse_prefill_workspace_size(int B, int Hq, int Hkv, int T) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || T < 0 || Hq % Hkv != 0) return 0;
  if (!items_fit(B, Hq, nqb_of(T))) return 0;
  const size_t entries = seer::sparse_work_entries(B, Hq, Hkv, nqb_of(T));
  return ((entries * sizeof(int32_t) + 255) / 256) * 256 + 256;
}

int seer_sparse_prefill_block(const void* q, const void* k, const void* v, int B, int Hq,
                              int Hkv, int T, int D, float sm_scale, int block,
                              const int32_t* kv_idx, const int32_t* kv_cnt, int max_k, void* o,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (block != 64 && block != 128) return SEER_ERR_UNSUPPORTED;
  const int st = attention_args(q, k, v, o, B, Hq, Hkv, T, D, sm_scale);
  if (st != SEER_OK) return st;
  if (max_k < 1) return SEER_ERR_INVALID_ARG;
  if ((long long)B * T == 0) return SEER_OK;
  if (!kv_idx || !kv_cnt) return SEER_ERR_INVALID_ARG;
  const size_t need = seer_sparse_prefill_workspace_size(B, Hq, Hkv, T);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return SEER_ERR_WORKSPACE;
  const hipError_t err =
      seer::launch_sparse_prefill(q, k, v, B, Hq, Hkv, T, D, sm_scale, block, kv_idx, kv_cnt,
                                  max_k, static_cast<int32_t*>(workspace), o, (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

int seer_sparse_prefill(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                        int T, int D, float sm_scale, const int32_t* kv_idx,
                        const int32_t* kv_cnt, int max_k, void* o, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return seer_sparse_prefill_block(q, k, v, B, Hq, Hkv, T, D, sm_scale, SEER_BLOCK, kv_idx,
                                   kv_cnt, max_k, o, workspace, workspace_bytes, stream);
}

int seer_sparse_prefill_noalloc(const void* q, const void* k, const void* v, int B, int Hq,
                                int Hkv, int T, int D, float sm_scale, const int32_t* kv_idx,
                                const int32_t* kv_cnt, int max_k, void* o, void* stream) {
  const int st = attention_args(q, k, v, o, B, Hq, Hkv, T, D, sm_scale);
  if (st != SEER_OK) return st;
  if (max_k < 1) return SEER_ERR_INVALID_ARG;
  if ((long long)B * T == 0) return SEER_OK;
  if (!kv_idx || !kv_cnt) return SEER_ERR_INVALID_ARG;
  if ((long long)B * Hq * nqb_of(T) > kNoAllocItems) return SEER_ERR_WORKSPACE;
  void* ws = nullptr;
  const int at = scratch_address(&ws);
  if (at != SEER_OK) return at;
  const hipError_t err =
      seer::launch_sparse_prefill(q, k, v, B, Hq, Hkv, T, D, sm_scale, SEER_BLOCK, kv_idx, kv_cnt,
                                  max_k, static_cast<int32_t*>(ws), o, (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

size_t seer_pooled_attn_map_workspace_size(int B, int Hq, int T) {
  if (B < 0 || Hq <= 0 || T < 0) return 0;
  const int nqb = nqb_of(T);
  if (!items_fit(B, Hq, nqb)) return 0;
  const size_t tiles = (size_t)B * Hq * ((size_t)nqb * (nqb + 1) / 2);
  return tiles * SEER_BLOCK * sizeof(float) + 256;
}

int seer_pooled_attn_map(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                         int T, int D, float sm_scale, void* o, float* amap, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const int st = attention_args(q, k, v, o, B, Hq, Hkv, T, D, sm_scale);
  if (st != SEER_OK) return st;
  if ((long long)B * T == 0) return SEER_OK;
  if (!amap) return SEER_ERR_INVALID_ARG;
  const size_t need = seer_pooled_attn_map_workspace_size(B, Hq, T);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return SEER_ERR_WORKSPACE;
  const hipError_t err =
      seer::launch_pooled_map(q, k, v, B, Hq, Hkv, T, D, sm_scale, o, amap,
                              static_cast<float*>(workspace), (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

int seer_pooled_target_mse(const float* amap, const float* gate, int B, int H, int nQB,
                           float* target, float* row_sse, float* loss, void* stream) {
  if (B < 0 || H < 0 || nQB < 0) return SEER_ERR_INVALID_ARG;
  if (!items_fit(B, H, nQB)) return SEER_ERR_UNSUPPORTED;
  if ((long long)B * H * nQB == 0) return SEER_OK;
  if (!amap || !target) return SEER_ERR_INVALID_ARG;
  if (loss && (!gate || !row_sse)) return SEER_ERR_INVALID_ARG;
  const hipError_t err = seer::launch_pooled_target(amap, gate, B, H, nQB, target,
                                                    gate ? row_sse : nullptr, gate ? loss : nullptr,
                                                    (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

size_t seer_attn_gate_workspace_size(int B, int Hq, int Hkv, int T, int Dg) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || T < 0 || Dg <= 0 || Hq % Hkv != 0) return 0;
  if (!items_fit(B, Hq + Hkv, nqb_of(T))) return 0;
  return seer::attn_gate_workspace_floats(B, Hq, Hkv, nqb_of(T), Dg) * sizeof(float) + 256;
}

int seer_attn_gate_scores(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                          const float* wq, const float* wk, int Dg, float scale, float rope_base,
                          float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return SEER_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SEER_ERR_UNSUPPORTED;
  if (Dg != 32 && Dg != 64 && Dg != 128) return SEER_ERR_UNSUPPORTED;
  if (!(isfinite(scale) && scale > 0.f)) return SEER_ERR_INVALID_ARG;
  if (!(isfinite(rope_base) && rope_base > 1.f)) return SEER_ERR_INVALID_ARG;
  if (!items_fit(B, Hq + Hkv, nqb_of(T))) return SEER_ERR_UNSUPPORTED;
  if ((long long)B * T == 0) return SEER_OK;
  if (!q || !k || !wq || !wk || !scores) return SEER_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(wq) || !aligned16(wk))
    return SEER_ERR_INVALID_ARG;
  const size_t need = seer_attn_gate_workspace_size(B, Hq, Hkv, T, Dg);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return SEER_ERR_WORKSPACE;
  const hipError_t err =
      seer::launch_attn_gate(q, k, B, Hq, Hkv, T, D, wq, wk, Dg, scale, rope_base, scores,
                             static_cast<float*>(workspace), (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

size_t seer_attn_gate_mask_workspace_size(int B, int Hq, int Hkv, int T, int Dg,
                                          int with_scores) {
  const size_t gate = seer_attn_gate_workspace_size(B, Hq, Hkv, T, Dg);
  if (gate == 0) return 0;
  const size_t nqb = (size_t)nqb_of(T);
  return gate + (with_scores ? 0 : (size_t)B * Hq * nqb * nqb * sizeof(float));
}

size_t seer_attn_gate_mask_pass_workspace_size(int B, int Hq, int Hkv, int T, int Dg,
                                               int pass_tiles) {
  const size_t gate = seer_attn_gate_workspace_size(B, Hq, Hkv, T, Dg);
  if (gate == 0 || pass_tiles < 1) return 0;
  const size_t nqb = (size_t)nqb_of(T);
  const size_t rows = std::min(nqb, (size_t)64 * (size_t)pass_tiles);
  return gate + (size_t)B * Hq * rows * nqb * sizeof(float);
}

int seer_attn_gate_mask(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                        const float* wq, const float* wk, int Dg, float scale, float rope_base,
                        int mode, float threshold, double density, int keep_sink,
                        int32_t* kv_idx, int32_t* kv_cnt, int max_k, float* scores,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return SEER_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SEER_ERR_UNSUPPORTED;
  if (Dg != 32 && Dg != 64 && Dg != 128) return SEER_ERR_UNSUPPORTED;
  if (!(isfinite(scale) && scale > 0.f)) return SEER_ERR_INVALID_ARG;
  if (!(isfinite(rope_base) && rope_base > 1.f)) return SEER_ERR_INVALID_ARG;
  const int nQB = nqb_of(T);
  if (nQB > SEER_MAX_QUERY_BLOCKS) return SEER_ERR_UNSUPPORTED;
  if (!items_fit(B, Hq + Hkv, nQB)) return SEER_ERR_UNSUPPORTED;
  if (mode != SEER_MASK_TOPK && mode != SEER_MASK_THRESHOLD) return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_TOPK && !(density > 0.0 && density <= 1.0)) return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_THRESHOLD && !isfinite(threshold)) return SEER_ERR_INVALID_ARG;
  if (max_k < 1) return SEER_ERR_CAPACITY;
  if ((long long)B * T == 0) return SEER_OK;
  if (!q || !k || !wq || !wk || !kv_idx || !kv_cnt) return SEER_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(wq) || !aligned16(wk))
    return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_TOPK) {
    if (max_k < seer_topk_budget(nQB, density, keep_sink)) return SEER_ERR_CAPACITY;
  } else {
    const int forced = (keep_sink && nQB > 1) ? 2 : 1;
    if (max_k < forced) return SEER_ERR_CAPACITY;
  }
  // Without scores the logits take what the workspace holds past the gate's own
  // part: all nQB rows per head (one pass), else whole tile rows of 64 (passes).
  const size_t gate = seer_attn_gate_workspace_size(B, Hq, Hkv, T, Dg);
  if (!workspace || workspace_bytes < gate || !aligned256(workspace)) return SEER_ERR_WORKSPACE;
  // Counted from the gate's full size (the logits start at or below it), so the
  // passes match seer_attn_gate_mask_pass_workspace_size exactly.
  int pass_rows = nQB;
  if (!scores) {
    const size_t row_bytes = (size_t)B * Hq * nQB * sizeof(float);
    const size_t fit = (workspace_bytes - gate) / row_bytes;
    if (fit < (size_t)nQB) pass_rows = (int)(fit / 64 * 64);
    if (pass_rows < 1) return SEER_ERR_WORKSPACE;
  }
  const hipError_t err = seer::launch_attn_gate_mask(
      q, k, B, Hq, Hkv, T, D, wq, wk, Dg, scale, rope_base, mode, threshold, density,
      keep_sink ? 1 : 0, kv_idx, kv_cnt, max_k, scores, static_cast<float*>(workspace),
      pass_rows, (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

namespace {

// Checks shared by the decode gate's workspace size and the call.
int decode_gate_sizes(int B, int Hq, int Hkv, int Tmax, int D, int Dg, int block) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Tmax < 1 || Hq % Hkv != 0) return SEER_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SEER_ERR_UNSUPPORTED;
  if (Dg != 32 && Dg != 64 && Dg != 128) return SEER_ERR_UNSUPPORTED;
  if (block != 64 && block != 128) return SEER_ERR_UNSUPPORTED;
  const long long nkb = (Tmax + (long long)block - 1) / block;
  if (nkb > SEER_MAX_QUERY_BLOCKS) return SEER_ERR_UNSUPPORTED;
  if (!items_fit(B, Hq > Hkv ? Hq : Hkv, nkb)) return SEER_ERR_UNSUPPORTED;
  return SEER_OK;
}

}  // namespace

size_t seer_attn_gate_decode_keys_workspace_size(int B, int Hkv, int Tmax, int D, int block) {
  if (decode_gate_sizes(B, Hkv, Hkv, Tmax, D, 32, block) != SEER_OK) return 0;
  const int nkb = (Tmax + block - 1) / block;
  return seer::attn_gate_decode_keys_workspace_floats(B, Hkv, nkb, D) * sizeof(float) + 256;
}

int seer_attn_gate_decode_keys(const void* k_cache, const int32_t* kv_len, int B, int Hkv,
                               int Tmax, int D, const float* wk, int Dg, float rope_base,
                               int block, int last_block_only, float* k_gate, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const int st = decode_gate_sizes(B, Hkv, Hkv, Tmax, D, Dg, block);
  if (st != SEER_OK) return st;
  if (!(isfinite(rope_base) && rope_base > 1.f)) return SEER_ERR_INVALID_ARG;
  if (B == 0) return SEER_OK;
  if (!k_cache || !kv_len || !wk || !k_gate) return SEER_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(wk)) return SEER_ERR_INVALID_ARG;
  if (!last_block_only) {  // only the all-block pass pools into the workspace
    const size_t need = seer_attn_gate_decode_keys_workspace_size(B, Hkv, Tmax, D, block);
    if (!workspace || workspace_bytes < need || !aligned256(workspace))
      return SEER_ERR_WORKSPACE;
  }
  const hipError_t err = seer::launch_attn_gate_decode_keys(
      k_cache, kv_len, B, Hkv, Tmax, D, wk, Dg, rope_base, block, last_block_only ? 1 : 0,
      k_gate, static_cast<float*>(workspace), (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

int seer_attn_gate_decode_scores(const void* q, const float* k_gate, const int32_t* kv_len,
                                 int B, int Hq, int Hkv, int Tmax, int D, const float* wq,
                                 int Dg, float scale, float rope_base, int block, float* scores,
                                 void* stream) {
  const int st = decode_gate_sizes(B, Hq, Hkv, Tmax, D, Dg, block);
  if (st != SEER_OK) return st;
  if (!(isfinite(scale) && scale > 0.f)) return SEER_ERR_INVALID_ARG;
  if (!(isfinite(rope_base) && rope_base > 1.f)) return SEER_ERR_INVALID_ARG;
  if (B == 0) return SEER_OK;
  if (!q || !k_gate || !kv_len || !wq || !scores) return SEER_ERR_INVALID_ARG;
  if (!aligned16(k_gate)) return SEER_ERR_INVALID_ARG;
  const hipError_t err = seer::launch_attn_gate_decode_scores(
      q, k_gate, kv_len, B, Hq, Hkv, Tmax, D, wq, Dg, scale, rope_base, block, scores,
      (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

int seer_attn_gate_decode_mask(const void* q, const float* k_gate, const int32_t* kv_len, int B,
                               int Hq, int Hkv, int Tmax, int D, const float* wq, int Dg,
                               float scale, float rope_base, int block, int mode,
                               float threshold, int k_blocks, int keep_sink, int32_t* kv_idx,
                               int32_t* kv_cnt, int max_k, float* scores, void* stream) {
  const int st = decode_gate_sizes(B, Hq, Hkv, Tmax, D, Dg, block);
  if (st != SEER_OK) return st;
  if (!(isfinite(scale) && scale > 0.f)) return SEER_ERR_INVALID_ARG;
  if (!(isfinite(rope_base) && rope_base > 1.f)) return SEER_ERR_INVALID_ARG;
  if (mode != SEER_MASK_TOPK && mode != SEER_MASK_THRESHOLD) return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_TOPK && k_blocks < 1) return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_THRESHOLD && !isfinite(threshold)) return SEER_ERR_INVALID_ARG;
  if (max_k < 1) return SEER_ERR_CAPACITY;
  const int nkb = (Tmax + block - 1) / block;
  const int forced = keep_sink ? 2 : 1;
  if (mode == SEER_MASK_TOPK) {
    const int want = k_blocks > forced ? k_blocks : forced;
    if (max_k < (want < nkb ? want : nkb)) return SEER_ERR_CAPACITY;
  } else {
    if (max_k < ((keep_sink && nkb > 1) ? 2 : 1)) return SEER_ERR_CAPACITY;
  }
  if ((long long)B * Hq * max_k > (long long)INT_MAX) return SEER_ERR_UNSUPPORTED;
  if (B == 0) return SEER_OK;
  if (!q || !k_gate || !kv_len || !wq || !kv_idx || !kv_cnt) return SEER_ERR_INVALID_ARG;
  if (!aligned16(k_gate)) return SEER_ERR_INVALID_ARG;
  const hipError_t err = seer::launch_attn_gate_decode_mask(
      q, k_gate, kv_len, B, Hq, Hkv, Tmax, D, wq, Dg, scale, rope_base, block, mode, threshold,
      k_blocks, keep_sink ? 1 : 0, kv_idx, kv_cnt, max_k, scores, (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

int seer_build_mask_decode(const float* scores, const int32_t* kv_len, int B, int H, int nKB,
                           int block, int mode, float threshold, int k_blocks, int keep_sink,
                           int32_t* kv_idx, int32_t* kv_cnt, int max_k, void* stream) {
  if (B < 0 || H < 0 || nKB < 0) return SEER_ERR_INVALID_ARG;
  if (block != 64 && block != 128) return SEER_ERR_UNSUPPORTED;
  if (nKB > SEER_MAX_QUERY_BLOCKS) return SEER_ERR_UNSUPPORTED;
  if (mode != SEER_MASK_TOPK && mode != SEER_MASK_THRESHOLD) return SEER_ERR_INVALID_ARG;
  if (!items_fit(B, H, 1)) return SEER_ERR_UNSUPPORTED;
  if (mode == SEER_MASK_TOPK && k_blocks < 1) return SEER_ERR_INVALID_ARG;
  if (mode == SEER_MASK_THRESHOLD && !isfinite(threshold)) return SEER_ERR_INVALID_ARG;
  if (max_k < 1) return SEER_ERR_CAPACITY;
  if ((long long)B * H == 0) return SEER_OK;
  if (!scores || !kv_len || !kv_idx || !kv_cnt) return SEER_ERR_INVALID_ARG;
  const int forced = keep_sink ? 2 : 1;
  if (mode == SEER_MASK_TOPK) {
    const int want = k_blocks > forced ? k_blocks : forced;
    if (max_k < (want < nKB ? want : nKB)) return SEER_ERR_CAPACITY;
  } else {
    if (max_k < ((keep_sink && nKB > 1) ? 2 : 1)) return SEER_ERR_CAPACITY;
  }
  const hipError_t err = seer::launch_build_mask_decode(
      scores, kv_len, B, H, nKB, block, mode, threshold, k_blocks, keep_sink ? 1 : 0, kv_idx,
      kv_cnt, max_k, (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

namespace {

// Checks shared by the decode workspace size and the decode call.
int decode_sizes(int B, int Hq, int Hkv, int Tmax, int D, int list_heads, int max_k, int block) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Tmax < 1 || max_k < 1) return SEER_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return SEER_ERR_INVALID_ARG;
  if (list_heads != Hq && list_heads != Hkv) return SEER_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SEER_ERR_UNSUPPORTED;
  if (block != 64 && block != 128) return SEER_ERR_UNSUPPORTED;
  if (Hq / Hkv > 8) return SEER_ERR_UNSUPPORTED;
  if ((Tmax + (long long)block - 1) / block > 32768) return SEER_ERR_UNSUPPORTED;
  if ((long long)B * Hq * max_k > (long long)INT_MAX) return SEER_ERR_UNSUPPORTED;
  if (seer::sparse_decode_grid(B, Hq, Hkv, Tmax, D, list_heads, max_k, block) > INT_MAX)
    return SEER_ERR_UNSUPPORTED;
  return SEER_OK;
}

}  // namespace

size_t seer_sparse_decode_workspace_size(int B, int Hq, int Hkv, int Tmax, int D,
                                         int list_heads, int max_k, int block) {
  if (decode_sizes(B, Hq, Hkv, Tmax, D, list_heads, max_k, block) != SEER_OK) return 0;
  return seer::sparse_decode_workspace_bytes(B, Hq, Hkv, Tmax, D, list_heads, max_k, block) +
         256;
}

int seer_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, int B, int Hq, int Hkv, int Tmax, int D,
                       float sm_scale, int block, const int32_t* kv_idx, const int32_t* kv_cnt,
                       int list_heads, int max_k, void* o, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const int st = decode_sizes(B, Hq, Hkv, Tmax, D, list_heads, max_k, block);
  if (st != SEER_OK) return st;
  if (!(isfinite(sm_scale) && sm_scale > 0.f)) return SEER_ERR_INVALID_ARG;
  if (B == 0) return SEER_OK;
  if (!q || !k_cache || !v_cache || !kv_len || !kv_idx || !kv_cnt || !o)
    return SEER_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return SEER_ERR_INVALID_ARG;
  const size_t need = seer_sparse_decode_workspace_size(B, Hq, Hkv, Tmax, D, list_heads, max_k,
                                                        block);
  if (!workspace || workspace_bytes < need || !aligned256(workspace)) return SEER_ERR_WORKSPACE;
  const hipError_t err = seer::launch_sparse_decode(q, k_cache, v_cache, kv_len, B, Hq, Hkv,
                                                    Tmax, D, sm_scale, block, kv_idx, kv_cnt,
                                                    list_heads, max_k, o, workspace,
                                                    (hipStream_t)stream);
  return err == hipSuccess ? SEER_OK : SEER_ERR_HIP;
}

}  // extern "C"
