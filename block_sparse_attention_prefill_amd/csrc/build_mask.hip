// Block-mask construction: fp32 soft block scores -> per-row ascending KV-block lists.
//
// Per-row TopK or threshold on the gate's soft scores (model card
// "SeerAttention-Llama-3.1-8B-AttnGates", method summary; TopK per row and the
// [Seq/Block, TopK] index layout from the rebuttal "SeerAttention: Learning
// Intrinsic Sparse Attention in Your LLMs", "Weakness 2 (Memory complexity)").
//
// Every candidate j <= i gets a 32-bit key that orders it exactly as the
// selection rule ranks it:
//   forced blocks (diagonal, optional block 0)  -> 0xFFFFFFFF (always first)
//   ranked candidates                           -> order-preserving image of the
//                                                  fp32 score (NaN as -inf, -0 as +0)
//   threshold mode, score below threshold       -> 0 (never selected)
// An 8-bit-digit radix select finds the k-th largest key t; ties on t are broken
// toward lower block indices by a running count in index order, which is also
// the output order, so each list comes out ascending without a sort.
//
// Decode rows (one per sequence and head, the new token's row) use the same
// rule over the blocks holding the sequence's kv_len tokens: the last of them,
// which holds the token itself, takes the diagonal's place, and TopK keeps a
// fixed number of blocks (a token budget over the block size) instead of a
// density of the row.
//
// One wave64 owns one row.  Row i's candidates sit in registers, candidate
// j = 64 * c + lane in slot c, so the score row is read from HBM once and the
// compaction is a ballot + popcount per 64 candidates.  The digit histograms
// live in a per-wave 1 KB slice of LDS.
#include "mask_select.h"

namespace seer {
namespace {

using rowsel::order_key;
using rowsel::wave_select_row;
using rowsel::wave_sum;

constexpr int kWavesPerGroup = 4;

// NPL = key slots per lane (row length <= 64 * NPL).
// One row by one wave, with NPL candidate slots per lane (rows of up to 64 NPL
// candidates).
template <int NPL>
__device__ __forceinline__ void mask_row(const float* __restrict__ srow, int i, int lane,
                                         int mode, float tau, double density, int keep_sink,
                                         int max_k, bool decode, int k_blocks, int* hist,
                                         int32_t* __restrict__ out, int32_t* __restrict__ cnt_out,
                                         int32_t* __restrict__ need_out) {
  const int n = i + 1;
  float sv[NPL];
  if (n > 0) {
#pragma unroll
    for (int c = 0; c < NPL; ++c) sv[c] = srow[min(64 * c + lane, i)];
  }
  uint32_t key[NPL];
  int npos = 0;
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    const int j = 64 * c + lane;
    uint32_t kj = 0u;
    if (j < n) {
      if (j == i || (keep_sink && j == 0)) {
        kj = 0xFFFFFFFFu;
      } else {
        const float s = sv[c];
        kj = (mode == 1 || s >= tau) ? order_key(s) : 0u;
      }
    }
    key[c] = kj;
    npos += kj != 0u;
  }
  npos = wave_sum(npos);

  int k;
  if (mode == 1) {
    const int forced = (i == 0) ? 1 : (keep_sink ? 2 : 1);
    const int want = decode ? k_blocks : (int)ceil(density * (double)(i + 1));
    k = min(i + 1, max(forced, want));
  } else {
    k = min(npos, max_k);
  }

  const int count = wave_select_row<NPL>(key, n, k, npos, lane, hist, out, max_k);
  if (lane == 0) {
    *cnt_out = count;
    if (need_out) *need_out = mode == 1 ? min(k, npos) : npos;
  }
}

// NPL = slots per lane the longest row of the launch needs; each wave takes the
// smallest slot count that holds its own row (the selection does not depend on
// it, so the lists are the same), so short rows skip the empty slots' work.
template <int NPL>
__global__ __launch_bounds__(64 * kWavesPerGroup) void build_mask_kernel(
    const float* __restrict__ scores, long long rows, int nqb, int nkb, int mode, float tau,
    double density, int keep_sink, int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
    int32_t* __restrict__ need, int max_k, const int32_t* __restrict__ kv_len, int heads,
    int block, int k_blocks) {
  __shared__ int hist_all[kWavesPerGroup][256];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * kWavesPerGroup + wv;
  if (row >= rows) return;
  int* hist = hist_all[wv];
  int i;  // last candidate block of the row (-1: no candidate)
  if (kv_len) {
    const int len = kv_len[row / heads];
    i = len > 0 ? min((len - 1) / block, nkb - 1) : -1;
  } else {
    i = (int)(row % nqb);
  }
  const float* srow = scores + row * (long long)nkb;
  int32_t* out = idx + row * (long long)max_k;
  int32_t* need_out = need ? need + row : nullptr;
  const bool decode = kv_len != nullptr;
#define SEER_MASK_ROW(P)                                                                   \
  mask_row<P>(srow, i, lane, mode, tau, density, keep_sink, max_k, decode, k_blocks, hist, \
              out, cnt + row, need_out)
  const int n = i + 1;
  if (NPL > 1 && n <= 64) {
    SEER_MASK_ROW(1);
  } else if (NPL > 4 && n <= 256) {
    SEER_MASK_ROW(4 < NPL ? 4 : NPL);
  } else if (NPL > 8 && n <= 512) {
    SEER_MASK_ROW(8 < NPL ? 8 : NPL);
  } else if (NPL > 16 && n <= 1024) {
    SEER_MASK_ROW(16 < NPL ? 16 : NPL);
  } else {
    SEER_MASK_ROW(NPL);
  }
#undef SEER_MASK_ROW
}

}  // namespace

namespace {

hipError_t launch_rows(const float* scores, long long rows, int nqb, int nkb, int row_len,
                       int mode, float threshold, double density, int keep_sink, int32_t* idx,
                       int32_t* cnt, int32_t* need, int max_k, const int32_t* kv_len, int heads,
                       int block, int k_blocks, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + kWavesPerGroup - 1) / kWavesPerGroup));
  const dim3 threads(64 * kWavesPerGroup);
#define SEER_MASK_LAUNCH(NPL)                                                                  \
  hipLaunchKernelGGL(build_mask_kernel<NPL>, grid, threads, 0, stream, scores, rows, nqb, nkb, \
                     mode, threshold, density, keep_sink, idx, cnt, need, max_k, kv_len,       \
                     heads, block, k_blocks)
  if (row_len <= 64 * 1) SEER_MASK_LAUNCH(1);
  else if (row_len <= 64 * 4) SEER_MASK_LAUNCH(4);
  else if (row_len <= 64 * 8) SEER_MASK_LAUNCH(8);
  else if (row_len <= 64 * 16) SEER_MASK_LAUNCH(16);
  else if (row_len <= 64 * 32) SEER_MASK_LAUNCH(32);
  else if (row_len <= 64 * 64) SEER_MASK_LAUNCH(64);
  else return hipErrorInvalidValue;  // the host layer rejects rows over 4096 blocks first
#undef SEER_MASK_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_mask(const float* scores, int B, int H, int nqb, int nkb, int mode,
                             float threshold, double density, int keep_sink, int32_t* idx,
                             int32_t* cnt, int32_t* need, int max_k, hipStream_t stream) {
  return launch_rows(scores, (long long)B * H * nqb, nqb, nkb, nqb, mode, threshold, density,
                     keep_sink, idx, cnt, need, max_k, nullptr, 1, 64, 0, stream);
}

hipError_t launch_build_mask_decode(const float* scores, const int32_t* kv_len, int B, int H,
                                    int nkb, int block, int mode, float threshold, int k_blocks,
                                    int keep_sink, int32_t* idx, int32_t* cnt, int max_k,
                                    hipStream_t stream) {
  return launch_rows(scores, (long long)B * H, 1, nkb, nkb, mode, threshold, 1.0, keep_sink, idx,
                     cnt, nullptr, max_k, kv_len, H, block, k_blocks, stream);
}

}  // namespace seer
