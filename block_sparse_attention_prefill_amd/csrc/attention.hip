// Block-sparse causal flash-attention prefill and the pooled-map pass for gfx950.
//
// Method: for each 64-row query block, visit only the selected 64-row KV blocks
// (K and V of a step share one block index) and keep an online softmax
// (running max m, running sum l, accumulator rescaled by alpha = exp(m_old -
// m_new)), dividing by l at the end (rebuttal "SeerAttention: Learning
// Intrinsic Sparse Attention in Your LLMs", "Weakness 5 (Pseudo code of
// Inference Kernel)"; its alpha line is read as exp(m_old - m_new), the
// standard flash-attention rescale).  The pooled-map variant visits every
// causal block, stores each tile's row maxima r_ij, and after the last block
// rescales them by the final m_i and l_i and takes the max over the tile's rows
// (reproducibility summary of "SeerAttention: Self-distilled Attention Gating
// for Efficient Long-context Prefilling", Pseudocode row, Figure 8).
//
// gfx950 mapping
// --------------
// * One workgroup = 2 wave64s = one (batch, head, query block).  Wave w owns
//   query rows 32w..32w+31 of the block.
// * Contractions use v_mfma_f32_32x32x16_bf16 in transposed form so that every
//   query row lives in one lane column:
//     S^T[kv][q] = K[kv][:] . Q[q][:]     (A = K tile from LDS, B = Q held in VGPRs)
//     O^T[d][q] += V^T[d][kv] . P^T[kv][q] (A = V^T tile from LDS, B = P^T straight
//                                          from the S^T accumulators)
//   Lane l then holds column q = l % 32 and half h = l / 32 of the rows, so a
//   row max or sum needs one cross-half exchange, and alpha and 1/l are
//   per-lane scalars.
// * The K tile sits in LDS row-major with a 16-byte row pad; V is stored
//   transposed (d-major) with a kv permutation inside each 16-key group that
//   makes every MFMA A-fragment one 16-byte LDS read and matches the register
//   order of P^T.  The transpose happens in registers on the way into LDS.
// * The next KV block's global loads are issued right after the current tile
//   is in LDS, so they are in flight during the two contractions.
// * exp2 with log2(e) folded into the softmax scale; fp32 row statistics.
#include "seer_internal.h"

#include <math.h>

namespace seer {
namespace {

constexpr int kThreads = 128;  // 2 waves
constexpr int kXcds = 8;       // MI355X: workgroups are dealt round-robin to 8 XCDs

template <int D>
struct Cfg {
  static constexpr int kKPitch = D + 8;            // bf16 per K row in LDS
  static constexpr int kVPitch = kBlk + 8;         // bf16 per V^T row in LDS
  static constexpr int kKSteps = D / 16;           // k-steps of the S^T contraction
  static constexpr int kDTiles = D / 32;           // 32-row tiles of O^T
  static constexpr int kChunks = D / 8;            // 16-byte chunks per K/V row
  static constexpr int kKLoads = kBlk * kChunks / kThreads;   // K chunks per thread
  static constexpr int kVGroups = 16 * kChunks / kThreads;    // (4 rows x 16 B) V groups per thread
  static constexpr int kLdsElems = kBlk * kKPitch + D * kVPitch;
};

// Position of key kv (0..63) inside a V^T row.  Within each group of 16 keys,
// key 8b + 4h + c goes to slot 8h + 4b + c, so the 8 keys a lane of half h
// needs for one PV k-step (its P^T register order) are contiguous.
__device__ __forceinline__ int vt_pos_of_quad(int kq) {
  return 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

template <int D>
struct KvStage {
  uint4 k[Cfg<D>::kKLoads];
  uint4 v[Cfg<D>::kVGroups][4];

  // Global -> registers for KV block starting at row `r0` of this head;
  // rows >= nvalid (short last block) read as zero.
  __device__ __forceinline__ void load(const __bf16* __restrict__ kh, const __bf16* __restrict__ vh,
                                       int r0, int nvalid, int tid) {
    const uint4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < Cfg<D>::kKLoads; ++m) {
      const int c = tid + kThreads * m;
      const int row = c / Cfg<D>::kChunks;
      const int col = c % Cfg<D>::kChunks;
      k[m] = (row < nvalid)
                 ? *reinterpret_cast<const uint4*>(kh + (size_t)(r0 + row) * D + col * 8)
                 : zero;
    }
#pragma unroll
    for (int m = 0; m < Cfg<D>::kVGroups; ++m) {
      const int g = tid + kThreads * m;
      const int kq = g & 15;
      const int dc = g >> 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * kq + e;
        v[m][e] = (row < nvalid)
                      ? *reinterpret_cast<const uint4*>(vh + (size_t)(r0 + row) * D + dc * 8)
                      : zero;
      }
    }
  }

  // Registers -> LDS: K row-major (padded), V transposed with the key permutation.
  __device__ __forceinline__ void store(__bf16* ks, __bf16* vt, int tid) const {
#pragma unroll
    for (int m = 0; m < Cfg<D>::kKLoads; ++m) {
      const int c = tid + kThreads * m;
      const int row = c / Cfg<D>::kChunks;
      const int col = c % Cfg<D>::kChunks;
      *reinterpret_cast<uint4*>(ks + row * Cfg<D>::kKPitch + col * 8) = k[m];
    }
#pragma unroll
    for (int m = 0; m < Cfg<D>::kVGroups; ++m) {
      const int g = tid + kThreads * m;
      const int kq = g & 15;
      const int dc = g >> 4;
      const int pos = vt_pos_of_quad(kq);
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&v[m][0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&v[m][1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&v[m][2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&v[m][3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint2 out;
        if (e & 1) {
          out.x = hi_pair(r0[w], r1[w]);
          out.y = hi_pair(r2[w], r3[w]);
        } else {
          out.x = lo_pair(r0[w], r1[w]);
          out.y = lo_pair(r2[w], r3[w]);
        }
        *reinterpret_cast<uint2*>(vt + (dc * 8 + e) * Cfg<D>::kVPitch + pos) = out;
      }
    }
  }
};

// Per-wave state of one query block: Q fragments, O^T accumulators, row stats.
template <int D>
struct RowState {
  bf16x8 qf[Cfg<D>::kKSteps];
  f32x16 acc[Cfg<D>::kDTiles];
  float m;  // running max of s * c (log2 domain)
  float l;  // this lane's partial row sum (its half of the keys)
};

struct BlockOut {
  float rowmax_raw;  // max of raw logits of this lane's query row in the tile
};

// One KV tile: S^T = K Q^T, causal mask on the diagonal tile, online softmax,
// O^T += V^T P^T.  Returns the raw row max (for the pooled map).
template <int D>
__device__ __forceinline__ float attend_tile(RowState<D>& st, const __bf16* ks, const __bf16* vt,
                                             int lane, int wave, bool diag, float c) {
  const int col = lane & 31;
  const int half = lane >> 5;
  f32x16 s[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    f32x16 a = {};
    const __bf16* krow = ks + (32 * tt + col) * Cfg<D>::kKPitch + 8 * half;
#pragma unroll
    for (int t = 0; t < Cfg<D>::kKSteps; ++t) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * t);
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, st.qf[t], a, 0, 0, 0);
    }
    s[tt] = a;
  }
  if (diag) {
    const int qrow = 32 * wave + col;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
        if (kv > qrow) s[tt][r] = -INFINITY;
      }
  }
  float mx = s[0][0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

  const float m_new = fmaxf(st.m, mx * c);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;
  float lsum = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[tt][r], c, -m_new));
      s[tt][r] = p;
      lsum += p;
    }
  st.l = st.l * alpha + lsum;
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[dt][r] *= alpha;

  // P^T fragments for the four 16-key steps: regs 8*(kk&1)..+7 of tile kk>>1.
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const f32x16& src = s[kk >> 1];
    const int o = 8 * (kk & 1);
    f32x8 pv = {src[o + 0], src[o + 1], src[o + 2], src[o + 3],
                src[o + 4], src[o + 5], src[o + 6], src[o + 7]};
    const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
    const __bf16* vrow = vt + col * Cfg<D>::kVPitch + 16 * kk + 8 * half;
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt) {
      const bf16x8 vf =
          *reinterpret_cast<const bf16x8*>(vrow + 32 * dt * Cfg<D>::kVPitch);
      st.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, st.acc[dt], 0, 0, 0);
    }
  }
  return mx;
}

template <int D>
__device__ __forceinline__ void load_q(RowState<D>& st, const __bf16* __restrict__ qh, int q0,
                                       int T, int lane, int wave) {
  const int row = q0 + 32 * wave + (lane & 31);
  const int half = lane >> 5;
#pragma unroll
  for (int t = 0; t < Cfg<D>::kKSteps; ++t) {
    if (row < T)
      st.qf[t] = *reinterpret_cast<const bf16x8*>(qh + (size_t)row * D + 16 * t + 8 * half);
    else
      st.qf[t] = bf16x8{};
  }
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt) st.acc[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
}

// O = acc / l, bf16 (RNE), rows >= T dropped.  Returns the full row sum.
template <int D>
__device__ __forceinline__ float store_o(const RowState<D>& st, __bf16* __restrict__ oh, int q0,
                                         int T, int lane, int wave) {
  const float l = st.l + __shfl_xor(st.l, 32, 64);
  const float inv = (l > 0.f) ? 1.0f / l : 0.f;
  const int row = q0 + 32 * wave + (lane & 31);
  const int half = lane >> 5;
  if (row < T) {
    __bf16* orow = oh + (size_t)row * D;
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 x = {st.acc[dt][4 * a + 0] * inv, st.acc[dt][4 * a + 1] * inv,
                   st.acc[dt][4 * a + 2] * inv, st.acc[dt][4 * a + 3] * inv};
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * a + 4 * half) = y;
      }
  }
  return l;
}

// ---------------------------------------------------------------------------
// Sparse prefill: one workgroup per scheduled (b, h, i).
template <int D>
__global__ __launch_bounds__(kThreads) void sparse_prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int Hq, int Hkv, int T, int nqb, float c, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, int max_k, const int32_t* __restrict__ work,
    __bf16* __restrict__ o) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[Cfg<D>::kLdsElems];
  __bf16* ks = lds;
  __bf16* vt = lds + kBlk * Cfg<D>::kKPitch;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int item = work[blockIdx.x];
  const int i = item % nqb;
  const int bh = item / nqb;  // b * Hq + h
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int g = h / (Hq / Hkv);
  const size_t kv_off = ((size_t)b * Hkv + g) * (size_t)T * D;
  const __bf16* kh = k + kv_off;
  const __bf16* vh = v + kv_off;
  const size_t q_off = (size_t)bh * (size_t)T * D;

  RowState<D> st;
  load_q<D>(st, q + q_off, kBlk * i, T, lane, wave);

  const int32_t* lst = idx + (size_t)item * max_k;
  const int n = min(max(cnt[item], 0), max_k);
  auto next_valid = [&](int e) {
    while (e < n) {
      const int j = lst[e];
      if (j >= 0 && j <= i) break;
      ++e;
    }
    return e;
  };

  KvStage<D> stage;
  int e = next_valid(0);
  int j = (e < n) ? lst[e] : -1;
  if (e < n) stage.load(kh, vh, kBlk * j, min(kBlk, T - kBlk * j), tid);
  while (e < n) {
    __syncthreads();
    stage.store(ks, vt, tid);
    __syncthreads();
    const int cur = j;
    e = next_valid(e + 1);
    if (e < n) {
      j = lst[e];
      stage.load(kh, vh, kBlk * j, min(kBlk, T - kBlk * j), tid);
    }
    (void)attend_tile<D>(st, ks, vt, lane, wave, cur == i, c);
  }
  (void)store_o<D>(st, o + q_off, kBlk * i, T, lane, wave);
}

// ---------------------------------------------------------------------------
// Pooled map: dense causal pass + per-tile row maxima, then the map row.
//
// Work order: heavy rows first (cost of row i is i + 1 tiles).  When the KV
// groups divide evenly over the 8 XCDs, all query heads of one KV group run on
// one XCD so that group's K/V stays in that XCD's L2.
__device__ __forceinline__ void pooled_item(int L, int B, int Hq, int Hkv, int nqb, int* b,
                                            int* h, int* i) {
  const int G = Hq / Hkv;
  const int ngroups = B * Hkv;
  if (ngroups % kXcds == 0) {
    const int xcd = L % kXcds;
    const int slot = L / kXcds;
    const int per_row = (ngroups / kXcds) * G;  // items of one query block on this XCD
    *i = nqb - 1 - slot / per_row;
    const int r = slot % per_row;
    const int grp = xcd + kXcds * (r / G);
    *b = grp / Hkv;
    *h = (grp % Hkv) * G + r % G;
  } else {
    const int per_row = B * Hq;
    *i = nqb - 1 - L / per_row;
    const int r = L % per_row;
    *b = r / Hq;
    *h = r % Hq;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void pooled_map_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int B, int Hq, int Hkv, int T, int nqb, float c, __bf16* __restrict__ o,
    float* __restrict__ amap, float* __restrict__ rws) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[Cfg<D>::kLdsElems];
  __shared__ float ms[kBlk];
  __shared__ float ils[kBlk];
  __bf16* ks = lds;
  __bf16* vt = lds + kBlk * Cfg<D>::kKPitch;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int b, h, i;
  pooled_item(blockIdx.x, B, Hq, Hkv, nqb, &b, &h, &i);
  const int g = h / (Hq / Hkv);
  const size_t bh = (size_t)b * Hq + h;
  const size_t kv_off = ((size_t)b * Hkv + g) * (size_t)T * D;
  const __bf16* kh = k + kv_off;
  const __bf16* vh = v + kv_off;
  const size_t q_off = bh * (size_t)T * D;
  // r_ij of this row block: packed lower triangle, 64 floats per tile.
  const size_t tri = (size_t)nqb * (nqb + 1) / 2;
  float* rrow = rws + (bh * tri + (size_t)i * (i + 1) / 2) * kBlk;

  RowState<D> st;
  load_q<D>(st, q + q_off, kBlk * i, T, lane, wave);

  KvStage<D> stage;
  stage.load(kh, vh, 0, min(kBlk, T), tid);
  for (int j = 0; j <= i; ++j) {
    __syncthreads();
    stage.store(ks, vt, tid);
    __syncthreads();
    if (j < i) stage.load(kh, vh, kBlk * (j + 1), min(kBlk, T - kBlk * (j + 1)), tid);
    const float mx = attend_tile<D>(st, ks, vt, lane, wave, j == i, c);
    if (lane < 32) rrow[(size_t)j * kBlk + 32 * wave + lane] = mx;
  }
  const float l = store_o<D>(st, o + q_off, kBlk * i, T, lane, wave);
  if (lane < 32) {
    const int r = 32 * wave + lane;
    const bool valid = kBlk * i + r < T;
    ms[r] = st.m;
    ils[r] = (valid && l > 0.f) ? 1.0f / l : 0.f;  // rows past T take no part in the max
  }
  __syncthreads();

  float* arow = amap + (bh * nqb + i) * (size_t)nqb;
  for (int j = tid; j <= i; j += kThreads) {
    const f32x4* rp = reinterpret_cast<const f32x4*>(rrow + (size_t)j * kBlk);
    float a = 0.f;
#pragma unroll 4
    for (int r4 = 0; r4 < kBlk / 4; ++r4) {
      const f32x4 x = rp[r4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * r4 + u;
        a = fmaxf(a, __builtin_amdgcn_exp2f(fmaf(x[u], c, -ms[r])) * ils[r]);
      }
    }
    arow[j] = a;
  }
  for (int j = i + 1 + tid; j < nqb; j += kThreads) arow[j] = 0.f;
}

// ---------------------------------------------------------------------------
// Schedule: order (b, h, i) items by descending block count (longest first),
// optionally grouping each KV head's items onto one XCD.  Single workgroup.
constexpr int kSchedThreads = 1024;
constexpr int kCostBins = 1024;

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    const int32_t* __restrict__ cnt, int B, int Hq, int Hkv, int nqb, int max_k,
    int32_t* __restrict__ work) {
  __shared__ int hist[kXcds][kCostBins];
  __shared__ int wsum[kSchedThreads / 64];
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const bool affinity = (B * Hkv) % kXcds == 0;
  const int nb = affinity ? kXcds : 1;
  const int n = B * Hq * nqb;
  for (int x = tid; x < kXcds * kCostBins; x += kSchedThreads) (&hist[0][0])[x] = 0;
  __syncthreads();
  auto bucket_of = [&](int item) {
    if (!affinity) return 0;
    const int bh = item / nqb;
    const int grp = (bh / Hq) * Hkv + (bh % Hq) / G;
    return grp % kXcds;
  };
  auto bin_of = [&](int item) {
    const int c = min(max(cnt[item], 0), max_k);
    return kCostBins - 1 - min(c, kCostBins - 1);  // bin 0 = most expensive
  };
  for (int it = tid; it < n; it += kSchedThreads) atomicAdd(&hist[bucket_of(it)][bin_of(it)], 1);
  __syncthreads();
  // Exclusive scan of each bucket's histogram (bin order = descending cost).
  const int lane = tid & 63, wv = tid >> 6;
  for (int bk = 0; bk < nb; ++bk) {
    const int v = hist[bk][tid];
    int incl = v;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    __syncthreads();
    hist[bk][tid] = before + incl - v;
    __syncthreads();
  }
  for (int it = tid; it < n; it += kSchedThreads) {
    const int bk = bucket_of(it);
    const int pos = atomicAdd(&hist[bk][bin_of(it)], 1);
    work[affinity ? pos * kXcds + bk : pos] = it;
  }
}

}  // namespace

hipError_t launch_schedule(const int32_t* cnt, int B, int Hq, int Hkv, int nqb, int max_k,
                           int32_t* work, hipStream_t stream) {
  if ((size_t)B * Hq * nqb == 0) return hipSuccess;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cnt, B, Hq, Hkv,
                     nqb, max_k, work);
  return hipGetLastError();
}

hipError_t launch_sparse_prefill(const void* q, const void* k, const void* v, int B, int Hq,
                                 int Hkv, int T, int D, float sm_scale, const int32_t* idx,
                                 const int32_t* cnt, int max_k, const int32_t* work, void* o,
                                 hipStream_t stream) {
  const int nqb = (T + kBlk - 1) / kBlk;
  const size_t items = (size_t)B * Hq * nqb;
  if (items == 0) return hipSuccess;
  const float c = sm_scale * 1.4426950408889634f;  // log2(e)
  const dim3 grid((unsigned)items), block(kThreads);
  if (D == 128)
    hipLaunchKernelGGL(sparse_prefill_kernel<128>, grid, block, 0, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, Hq, Hkv, T, nqb, c, idx, cnt, max_k,
                       work, (__bf16*)o);
  else
    hipLaunchKernelGGL(sparse_prefill_kernel<64>, grid, block, 0, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, Hq, Hkv, T, nqb, c, idx, cnt, max_k,
                       work, (__bf16*)o);
  return hipGetLastError();
}

hipError_t launch_pooled_map(const void* q, const void* k, const void* v, int B, int Hq,
                             int Hkv, int T, int D, float sm_scale, void* o, float* amap,
                             float* rowmax_ws, hipStream_t stream) {
  const int nqb = (T + kBlk - 1) / kBlk;
  const size_t items = (size_t)B * Hq * nqb;
  if (items == 0) return hipSuccess;
  const float c = sm_scale * 1.4426950408889634f;
  const dim3 grid((unsigned)items), block(kThreads);
  if (D == 128)
    hipLaunchKernelGGL(pooled_map_kernel<128>, grid, block, 0, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, B, Hq, Hkv, T, nqb, c, (__bf16*)o,
                       amap, rowmax_ws);
  else
    hipLaunchKernelGGL(pooled_map_kernel<64>, grid, block, 0, stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, B, Hq, Hkv, T, nqb, c, (__bf16*)o,
                       amap, rowmax_ws);
  return hipGetLastError();
}

}  // namespace seer
