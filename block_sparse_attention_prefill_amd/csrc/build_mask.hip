// Block-mask construction: fp32 soft block scores -> per-row ascending KV-block lists.
//
// Per-row TopK or threshold on the gate's soft scores (model card
// "SeerAttention-Llama-3.1-8B-AttnGates", method summary; TopK per row and the
// [Seq/Block, TopK] index layout from the rebuttal "SeerAttention: Learning
// Intrinsic Sparse Attention in Your LLMs", "Weakness 2 (Memory complexity)").
//
// One 256-thread workgroup owns one row (b, h, i).  Every candidate j <= i gets
// a 32-bit key that orders it exactly as the selection rule ranks it:
//   forced blocks (diagonal, optional block 0)  -> 0xFFFFFFFF (always first)
//   ranked candidates                           -> order-preserving image of the
//                                                  fp32 score (NaN as -inf, -0 as +0)
//   threshold mode, score below threshold       -> 0 (never selected)
// A 4-pass, 8-bit radix select finds the k-th largest key t; ties on t are
// broken toward lower block indices by a prefix count in index order, which is
// also the output order, so the list comes out ascending without a sort.
#include "seer_internal.h"

namespace seer {
namespace {

constexpr int kMaskThreads = 256;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) u = 0xFF800000u;   // NaN ranks as -inf
  if (u == 0x80000000u) u = 0u;  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; *total receives the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* lds4) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) lds4[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kMaskThreads / 64; ++w) {
    int t = lds4[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__global__ __launch_bounds__(kMaskThreads) void build_mask_kernel(
    const float* __restrict__ scores, int nqb, int nkb, int mode, float tau, double density,
    int keep_sink, int32_t* __restrict__ idx, int32_t* __restrict__ cnt, int max_k) {
  __shared__ int hist[256];
  __shared__ int lds4[kMaskThreads / 64];
  __shared__ int sel_bin, sel_above;

  const size_t row = blockIdx.x;
  const int i = (int)(row % (size_t)nqb);
  const int n = i + 1;
  const int tid = threadIdx.x;
  const float* srow = scores + row * (size_t)nkb;
  int32_t* out = idx + row * (size_t)max_k;

  auto key_of = [&](int j) -> uint32_t {
    if (j == i || (keep_sink && j == 0)) return 0xFFFFFFFFu;
    const float s = srow[j];
    if (mode == 1) return order_key(s);
    return (s >= tau) ? order_key(s) : 0u;
  };

  int npos_local = 0;
  for (int j = tid; j < n; j += kMaskThreads) npos_local += key_of(j) != 0u;
  int npos;
  (void)block_excl_scan(npos_local, &npos, lds4);

  int k;
  if (mode == 1) {
    const int forced = (i == 0) ? 1 : (keep_sink ? 2 : 1);
    const double c = ceil(density * (double)(i + 1));
    k = min(i + 1, max(forced, (int)c));
  } else {
    k = min(npos, max_k);
  }

  // Keys > t are kept, and the first `need` keys equal to t in index order.
  uint32_t t = 0u;
  int need = 0;
  if (k < npos) {
    uint32_t prefix = 0u, mask = 0u;
    int remaining = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < n; j += kMaskThreads) {
        const uint32_t kj = key_of(j);
        if ((kj & mask) == prefix) atomicAdd(&hist[(kj >> shift) & 255u], 1);
      }
      __syncthreads();
      // Thread tid looks at bin 255 - tid: running count from the top bin down.
      const int c = hist[255 - tid];
      int tot;
      const int excl = block_excl_scan(c, &tot, lds4);
      if (excl < remaining && remaining <= excl + c) {
        sel_bin = 255 - tid;
        sel_above = excl;
      }
      __syncthreads();
      prefix |= (uint32_t)sel_bin << shift;
      mask |= 0xFFu << shift;
      remaining -= sel_above;
      __syncthreads();
    }
    t = prefix;
    need = remaining;
  }

  int base = 0, ties = 0;
  for (int j0 = 0; j0 < n; j0 += kMaskThreads) {
    const int j = j0 + tid;
    const uint32_t kj = (j < n) ? key_of(j) : 0u;
    const bool eq = (j < n) && (kj == t);
    int eq_tot;
    const int eq_rank = ties + block_excl_scan(eq ? 1 : 0, &eq_tot, lds4);
    ties += eq_tot;
    const bool keep = (j < n) && (kj > t || (eq && eq_rank < need));
    int kept;
    const int pos = base + block_excl_scan(keep ? 1 : 0, &kept, lds4);
    if (keep) out[pos] = j;
    base += kept;
  }
  for (int p = base + tid; p < max_k; p += kMaskThreads) out[p] = -1;
  if (tid == 0) cnt[row] = base;
}

}  // namespace

hipError_t launch_build_mask(const float* scores, int B, int H, int nqb, int nkb, int mode,
                             float threshold, double density, int keep_sink, int32_t* idx,
                             int32_t* cnt, int max_k, hipStream_t stream) {
  const size_t rows = (size_t)B * H * nqb;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(build_mask_kernel, dim3((unsigned)rows), dim3(kMaskThreads), 0, stream,
                     scores, nqb, nkb, mode, threshold, density, keep_sink, idx, cnt, max_k);
  return hipGetLastError();
}

}  // namespace seer
