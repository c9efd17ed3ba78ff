// List validation: checks block lists against what the sparse prefill and
// decode calls require of them and reports every violation as a flag bit.
//
// The lists are the per-row [Seq/Block, TopK] block indices of the rebuttal
// "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs", "Weakness 2
// (Memory complexity)".  The prefill skips entries outside [0, i] and reads a
// count above max_k as max_k, so neither corrupts memory; a repeated block,
// however, would be accumulated twice, and a threshold row cut to max_k
// (model card "SeerAttention-Llama-3.1-8B-AttnGates", method summary:
// threshold on the soft scores) silently differs from what the threshold
// selects.  This pass makes both visible.
//
// One wave64 per list row.  The row's entries are read 64 at a time; each lane
// compares its entry with the previous one (order and, for ascending lists,
// repeats) and marks it in a per-wave LDS bitmap of the row's causal blocks,
// which catches repeats in any order for rows of up to kBitmapBlocks blocks.
#include "seer_internal.h"

#include <limits.h>

#include "seer.h"

namespace seer {
namespace {

constexpr int kValWaves = 4;
constexpr int kBitmapBlocks = 8192;  // bits per wave: 1 KB of LDS

__global__ __launch_bounds__(64) void clear_flags_kernel(int32_t* flags) {
  if (threadIdx.x == 0) flags[0] = 0;
}

__global__ __launch_bounds__(64 * kValWaves) void validate_lists_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ need, long long rows, int nrows_per_head, int max_k,
    int32_t* __restrict__ row_flags, int32_t* __restrict__ flags) {
  __shared__ uint32_t bitmap_all[kValWaves][kBitmapBlocks / 32];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * kValWaves + wv;
  if (row >= rows) return;
  uint32_t* bitmap = bitmap_all[wv];
  const int i = (int)(row % nrows_per_head);  // the row's own (diagonal) block
  const int c = cnt[row];
  int f = 0;
  if (c < 0 || c > max_k) f |= SEER_LIST_BAD_COUNT;
  if (need && need[row] > max_k) f |= SEER_LIST_CAPACITY;
  const int n = min(max(c, 0), max_k);
  const bool use_bitmap = i < kBitmapBlocks;
  if (use_bitmap)
    for (int w = lane; w <= i / 32; w += 64) bitmap[w] = 0u;
  __builtin_amdgcn_wave_barrier();
  const int32_t* lst = idx + row * (long long)max_k;
  int carry = INT_MIN;  // the entry before this chunk
  for (int b = 0; b < n; b += 64) {
    const int x = b + lane;
    const bool in = x < n;
    const int e = in ? lst[x] : 0;
    int prev = __shfl_up(e, 1, 64);
    if (lane == 0) prev = carry;
    if (in) {
      const bool ok = e >= 0 && e <= i;
      if (!ok) {
        f |= SEER_LIST_BAD_ENTRY;  // skipped by the calls, so never a repeat
      } else if (use_bitmap) {
        const uint32_t bit = 1u << (e & 31);
        if (atomicOr(&bitmap[e >> 5], bit) & bit) f |= SEER_LIST_REPEAT;
      }
      if (x > 0 && e <= prev) {
        f |= SEER_LIST_UNSORTED;
        if (ok && e == prev) f |= SEER_LIST_REPEAT;
      }
    }
    carry = __shfl(e, 63, 64);
  }
  // OR over the wave, then one atomic per row with a violation.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) f |= __shfl_xor(f, off, 64);
  if (lane == 0) {
    if (row_flags) row_flags[row] = f;
    if (f) atomicOr(flags, f);
  }
}

}  // namespace

hipError_t launch_validate_lists(const int32_t* idx, const int32_t* cnt, const int32_t* need,
                                 long long rows, int nrows_per_head, int max_k,
                                 int32_t* row_flags, int32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(64), 0, stream, flags);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || rows == 0) return err;
  const dim3 grid((unsigned)((rows + kValWaves - 1) / kValWaves));
  hipLaunchKernelGGL(validate_lists_kernel, grid, dim3(64 * kValWaves), 0, stream, idx, cnt, need,
                     rows, nrows_per_head, max_k, row_flags, flags);
  return hipGetLastError();
}

}  // namespace seer
