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
// * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4, no
//   register staging), in their natural [key][d] layout with XOR-swizzled
//   16-byte chunks.  K fragments are plain 16-byte LDS reads; V^T fragments come
//   from ds_read_b64_tr_b16, which transposes 4x16 bf16 blocks on the fly into
//   the key order of P^T's registers.
// * K and V of a tile are separate pipeline stages: K(j+1) streams in during
//   softmax and PV of tile j, V(j+1) during QK of tile j+1.
// * exp2 with log2(e) folded into the softmax scale; fp32 row statistics; the
//   reference max is raised lazily (only when a tile exceeds it by 2^8), which
//   leaves O = acc / l unchanged and skips most accumulator rescales.
#include "seer_internal.h"

#include <math.h>

namespace seer {
namespace {

constexpr int kThreads = 128;  // 2 waves
constexpr int kXcds = 8;       // MI355X: workgroups are dealt round-robin to 8 XCDs
// The running row max is only raised when a tile's max exceeds it by more than
// this many powers of two; P values stay <= 2^8 and both O and l use the same
// reference max, so the result is unchanged while most tiles skip the rescale.
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct Cfg {
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int kRowsPerLoad = 64 / kChunks;      // rows per 1 KB wave-wide LDS load
  static constexpr int kLoadsPerTile = kBlk / kRowsPerLoad;
  static constexpr int kLoadsPerWave = kLoadsPerTile / 2;
  static constexpr int kKSteps = D / 16;                 // k-steps of the S^T contraction
  static constexpr int kDTiles = D / 32;                 // 32-row tiles of O^T
  // LDS tile layout: slab n (one 1 KB wave-wide copy) holds rows n, n + S,
  // n + 2S, ... (S = kLoadsPerTile slabs per tile), each row whole and in order,
  // so every 16-lane group of a copy reads one contiguous row from HBM.  Slabs
  // are spaced by a padded stride so that the rows read together land on
  // distinct LDS banks: 16 rows at one 16-byte chunk for K (stride = 1 KB + 16 B,
  // rows step by 4 banks), 4 rows x 4 chunks for the V transpose reads (stride =
  // 1 KB + 64 B, rows step by 16 banks).
  static constexpr int kKSlab = 1024 + 16;
  static constexpr int kVSlab = 1024 + 64;
  static constexpr int kKTileBytes = kLoadsPerTile * kKSlab;
  static constexpr int kVTileBytes = kLoadsPerTile * kVSlab;
};

// Byte offset of (row, 16-byte chunk) inside a K or V tile in LDS.
template <int D, bool IS_V>
__device__ __forceinline__ int tile_byte(int row, int chunk) {
  constexpr int S = Cfg<D>::kLoadsPerTile;
  return (row % S) * (IS_V ? Cfg<D>::kVSlab : Cfg<D>::kKSlab) + (row / S) * (2 * D) + 16 * chunk;
}

#define SEER_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  compiler_fence();
}

__device__ __forceinline__ void wg_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Barrier after which a tile may be overwritten: this wave's LDS reads of it
// have returned (lgkmcnt(0)) before any wave passes.
__device__ __forceinline__ void wg_barrier_reads_done() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4));  // lgkmcnt(0), other counters free
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// One wave-wide HBM -> LDS copy: every lane moves 16 bytes from sbase + voff
// (its own byte offset) to lds_base + 16 * lane (global_load_lds_dwordx4 in
// its SGPR-base form; M0 holds the LDS base).  Written as inline asm so that
// the compiler does not add conservative vmcnt(0) waits in front of unrelated
// LDS reads; every copy is instead waited for explicitly with wait_vmcnt<>
// before a barrier, and each one is consumed before the kernel ends.  The
// instruction writes no VGPR.
__device__ __forceinline__ uint64_t uniform_u64(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t lds_u32(const char* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p));
}

__device__ __forceinline__ void dma16(uint64_t sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "memory");
}

// Per-lane HBM byte offsets of this wave's share of one 64-row tile: slab n of
// wave w is slab w * NL + n; its lane L copies chunk L % chunks of row
// slab + S * (L / chunks).  Rows at or past `nvalid` (short last block) re-read
// the last valid row; those keys are always causally masked, and no LDS slot is
// left stale.
template <int D>
__device__ __forceinline__ void tile_offsets(uint32_t (&off)[Cfg<D>::kLoadsPerWave], int nvalid,
                                             int wave, int lane) {
  const int r = lane / Cfg<D>::kChunks;
  const int ch = lane % Cfg<D>::kChunks;
#pragma unroll
  for (int n = 0; n < Cfg<D>::kLoadsPerWave; ++n) {
    const int row = (wave * Cfg<D>::kLoadsPerWave + n) + Cfg<D>::kLoadsPerTile * r;
    const int grow = row < nvalid ? row : nvalid - 1;
    off[n] = (uint32_t)((grow * D + ch * 8) * 2);
  }
}

template <int D>
struct TileIssue {
  uint32_t off[Cfg<D>::kLoadsPerWave];
  uint32_t kbase_lds, vbase_lds;  // LDS byte address of this wave's first slab
  __device__ __forceinline__ void init(const char* ks, const char* vs, int wave, int lane) {
    tile_offsets<D>(off, kBlk, wave, lane);
    kbase_lds = lds_u32(ks) + wave * Cfg<D>::kLoadsPerWave * Cfg<D>::kKSlab;
    vbase_lds = lds_u32(vs) + wave * Cfg<D>::kLoadsPerWave * Cfg<D>::kVSlab;
  }
  // Issue this wave's share of a tile (K or V) whose first row is `g`.
  template <bool IS_V>
  __device__ __forceinline__ void issue(const __bf16* g, int nvalid, int wave, int lane) const {
    const uint64_t sb = uniform_u64(g);
    const uint32_t lb = IS_V ? vbase_lds : kbase_lds;
    constexpr uint32_t stride = IS_V ? Cfg<D>::kVSlab : Cfg<D>::kKSlab;
    if (nvalid >= kBlk) {
#pragma unroll
      for (int n = 0; n < Cfg<D>::kLoadsPerWave; ++n) dma16(sb, off[n], lb + n * stride);
    } else {
      uint32_t o[Cfg<D>::kLoadsPerWave];
      tile_offsets<D>(o, nvalid, wave, lane);
#pragma unroll
      for (int n = 0; n < Cfg<D>::kLoadsPerWave; ++n) dma16(sb, o[n], lb + n * stride);
    }
  }
};

// Per-wave state of one query block: Q fragments, O^T accumulators, row stats.
template <int D>
struct RowState {
  bf16x8 qf[Cfg<D>::kKSteps];
  f32x16 acc[Cfg<D>::kDTiles];
  float m;  // reference max of s * c (log2 domain)
  float l;  // this lane's partial row sum (its half of the keys)
};

// S^T = K Q^T for one 64-key tile (two 32-key MFMA tiles), causal mask on the
// diagonal tile.  Reads the K tile from LDS; all fragments of a 32-key tile
// are requested before its MFMAs so the LDS latency is paid once.
template <int D>
__device__ __forceinline__ void qk_tile(const RowState<D>& st, const char* ks, int lane, int wave,
                                        bool diag, f32x16 (&s)[2]) {
  const int col = lane & 31;
  const int half = lane >> 5;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const char* krow = ks + tile_byte<D, false>(32 * tt + col, half);
    bf16x8 kf[Cfg<D>::kKSteps];
#pragma unroll
    for (int t = 0; t < Cfg<D>::kKSteps; ++t)
      kf[t] = *reinterpret_cast<const bf16x8*>(krow + 32 * t);
    f32x16 a = {};
#pragma unroll
    for (int t = 0; t < Cfg<D>::kKSteps; ++t)
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], st.qf[t], a, 0, 0, 0);
    s[tt] = a;
  }
  if (diag) {  // wave-uniform; the fence keeps it a branch instead of 32 selects per tile
    compiler_fence();
    const int qrow = 32 * wave + col;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kv = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
        if (kv > qrow) s[tt][r] = -INFINITY;
      }
  }
}

// v_max3_f32 directly: fmaxf chains on MFMA results otherwise get an extra
// canonicalising v_max per element.  Inputs are finite or -inf (never NaN).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Online softmax update on S^T (in place -> P), returns the raw row max.
// EXACT_L: accumulate l from the fp32 probabilities here (the pooled map needs
// l to fp32 accuracy); otherwise pv_tile sums the bf16 probabilities it feeds
// to the MFMA, so numerator and denominator use the same weights.
template <int D, bool EXACT_L>
__device__ __forceinline__ float softmax_tile(RowState<D>& st, f32x16 (&s)[2], float c) {
  float m0 = max3f(s[0][0], s[0][1], s[0][2]);
  float m1 = max3f(s[1][0], s[1][1], s[1][2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) {
    m0 = max3f(m0, s[0][r], s[0][r + 1]);
    m1 = max3f(m1, s[1][r], s[1][r + 1]);
  }
  float mx = max3f(m0, m1, max3f(s[0][15], s[1][15], -INFINITY));
  mx = max3f(mx, __shfl_xor(mx, 32, 64), -INFINITY);

  const float cand = mx * c;
  const bool raise = cand > st.m + kRescaleSlack;
  if (__any(raise)) {
    const float m_new = raise ? cand : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[dt][r] *= alpha;
  }
  const float nm = -st.m;
  float lsum = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[tt][r], c, nm));
      s[tt][r] = p;
      if (EXACT_L) lsum += p;
    }
  if (EXACT_L) st.l += lsum;
  return mx;
}

// O^T += V^T P^T.  The V tile sits in LDS in its natural [key][d] layout;
// ds_read_b64_tr_b16 hands each lane four consecutive keys of one d, which is
// exactly the A-fragment order matching P^T's registers.
template <int D, bool EXACT_L>
__device__ __forceinline__ void pv_tile(RowState<D>& st, const f32x16 (&s)[2], const char* vs,
                                        int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
  const int g = lane >> 4;
  const int i = lane & 15;
  const int h = g >> 1;
  const int r = i >> 2;
  const int sub = 4 * (i & 1);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float lsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int kv_a = 16 * kk + 4 * h + r;
    const int kv_b = kv_a + 8;
    const char* va_row = vs + tile_byte<D, true>(kv_a, 2 * (g & 1) + ((i & 3) >> 1)) + 2 * sub;
    const char* vb_row = vs + tile_byte<D, true>(kv_b, 2 * (g & 1) + ((i & 3) >> 1)) + 2 * sub;
    s16x4 va[Cfg<D>::kDTiles], vb[Cfg<D>::kDTiles];
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt) {
      va[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(va_row + 64 * dt));
      vb[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vb_row + 64 * dt));
    }
    const f32x16& src = s[kk >> 1];
    const int o = 8 * (kk & 1);
    const f32x8 pv = {src[o + 0], src[o + 1], src[o + 2], src[o + 3],
                      src[o + 4], src[o + 5], src[o + 6], src[o + 7]};
    const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
    if (!EXACT_L) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x2 pair = {pb[2 * u], pb[2 * u + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lsum, false);
      }
    }
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt) {
      const s16x8 vv = {va[dt][0], va[dt][1], va[dt][2], va[dt][3],
                        vb[dt][0], vb[dt][1], vb[dt][2], vb[dt][3]};
      st.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb,
                                                           st.acc[dt], 0, 0, 0);
    }
  }
  if (!EXACT_L) st.l += lsum;
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

// The KV-block loop shared by both kernels.  Tile j's K and V are loaded in
// separate stages so that K(j+1) streams in during softmax + PV of tile j and
// V(j+1) during QK of tile j+1.  `next(e)` returns the next list position and
// `block(e)` its KV block; `on_tile(j, rowmax)` observes every tile.
// The query fragments are loaded after the first tile's copies are issued and
// everything is drained once before the loop, so Q's latency overlaps the first
// tile's and the loop body never waits on an older load.
template <int D, bool EXACT_L, typename Next, typename Block, typename OnTile>
__device__ __forceinline__ void kv_loop(RowState<D>& st, const __bf16* __restrict__ qh, int q0,
                                        const __bf16* __restrict__ kh,
                                        const __bf16* __restrict__ vh, int T, int i, int n,
                                        Next next, Block block, OnTile on_tile, char* ks,
                                        char* vs, int lane, int wave, float c) {
  constexpr int NL = Cfg<D>::kLoadsPerWave;
  int e = next(0);
  if (e >= n) {
    load_q<D>(st, qh, q0, T, lane, wave);
    return;
  }
  TileIssue<D> io;
  io.init(ks, vs, wave, lane);
  int j = block(e);
  io.template issue<false>(kh + (size_t)kBlk * j * D, T - kBlk * j, wave, lane);
  io.template issue<true>(vh + (size_t)kBlk * j * D, T - kBlk * j, wave, lane);
  load_q<D>(st, qh, q0, T, lane, wave);
  wait_vmcnt<0>();
  while (true) {
    const int cur = j;
    e = next(e + 1);
    const bool more = e < n;
    if (more) j = block(e);

    wait_vmcnt<NL>();  // K(cur) has landed; V(cur) may still be in flight
    wg_barrier();
    f32x16 s[2];
    qk_tile<D>(st, ks, lane, wave, cur == i, s);
    wg_barrier_reads_done();  // every wave is done reading K(cur)
    if (more) io.template issue<false>(kh + (size_t)kBlk * j * D, T - kBlk * j, wave, lane);
    const float mx = softmax_tile<D, EXACT_L>(st, s, c);
    on_tile(cur, mx);
    if (more) wait_vmcnt<NL>(); else wait_vmcnt<0>();  // V(cur) has landed
    wg_barrier();
    pv_tile<D, EXACT_L>(st, s, vs, lane);
    wg_barrier_reads_done();  // every wave is done reading V(cur)
    if (!more) break;
    io.template issue<true>(vh + (size_t)kBlk * j * D, T - kBlk * j, wave, lane);
  }
}

// ---------------------------------------------------------------------------
// Sparse prefill: one workgroup per scheduled (b, h, i).
template <int D>
__global__ __launch_bounds__(kThreads, 2) void sparse_prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int Hq, int Hkv, int T, int nqb, float c, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, int max_k, const int32_t* __restrict__ work,
    __bf16* __restrict__ o) {
  __shared__ __attribute__((aligned(1024))) char ks[Cfg<D>::kKTileBytes];
  __shared__ __attribute__((aligned(1024))) char vs[Cfg<D>::kVTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = work[blockIdx.x];
  const int i = item % nqb;
  const int bh = item / nqb;  // b * Hq + h
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int g = h / (Hq / Hkv);
  const size_t kv_off = ((size_t)b * Hkv + g) * (size_t)T * D;
  const size_t q_off = (size_t)bh * (size_t)T * D;

  RowState<D> st;
  const int32_t* lst = idx + (size_t)item * max_k;
  const int n = min(max(cnt[item], 0), max_k);
  auto next = [&](int e) {
    while (e < n) {
      const int j = lst[e];
      if (j >= 0 && j <= i) break;
      ++e;
    }
    return e;
  };
  auto block = [&](int e) { return lst[e]; };
  auto on_tile = [](int, float) {};
  kv_loop<D, false>(st, q + q_off, kBlk * i, k + kv_off, v + kv_off, T, i, n, next, block, on_tile, ks,
             vs, lane, wave, c);
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
__global__ __launch_bounds__(kThreads, 2) void pooled_map_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int B, int Hq, int Hkv, int T, int nqb, float c, __bf16* __restrict__ o,
    float* __restrict__ amap, float* __restrict__ rws) {
  __shared__ __attribute__((aligned(1024))) char ks[Cfg<D>::kKTileBytes];
  __shared__ __attribute__((aligned(1024))) char vs[Cfg<D>::kVTileBytes];
  __shared__ float ms[kBlk];
  __shared__ float ils[kBlk];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b, h, i;
  pooled_item(blockIdx.x, B, Hq, Hkv, nqb, &b, &h, &i);
  const int g = h / (Hq / Hkv);
  const size_t bh = (size_t)b * Hq + h;
  const size_t kv_off = ((size_t)b * Hkv + g) * (size_t)T * D;
  const size_t q_off = bh * (size_t)T * D;
  // r_ij of this row block: packed lower triangle, 64 floats per tile.
  const size_t tri = (size_t)nqb * (nqb + 1) / 2;
  float* rrow = rws + (bh * tri + (size_t)i * (i + 1) / 2) * kBlk;

  RowState<D> st;
  auto next = [](int e) { return e; };
  auto block = [](int e) { return e; };
  auto on_tile = [&](int j, float mx) {
    if (lane < 32) rrow[(size_t)j * kBlk + 32 * wave + lane] = mx;
  };
  kv_loop<D, true>(st, q + q_off, kBlk * i, k + kv_off, v + kv_off, T, i, i + 1, next, block, on_tile,
             ks, vs, lane, wave, c);
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
// Schedule (longest-processing-time first): one workgroup per KV group
// (b, g) counting-sorts that group's G * nQB query-block items by descending
// list length; the rank-r item of group q goes to position r * NG + q of the
// work list.  Workgroups are dispatched in position order, so long rows start
// first everywhere; and since the hardware deals workgroup L to XCD L % 8,
// every item of a group lands on the same XCD whenever NG is a multiple of 8
// (its K/V then stays in that XCD's L2).
constexpr int kSchedThreads = 1024;
constexpr int kCostBins = 1024;

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    const int32_t* __restrict__ cnt, int Hq, int Hkv, int nqb, int max_k,
    int32_t* __restrict__ work) {
  __shared__ int hist[kCostBins];
  __shared__ int wsum[kSchedThreads / 64];
  const int tid = threadIdx.x;
  const int ng = gridDim.x;
  const int grp = blockIdx.x;
  const int G = Hq / Hkv;
  const int b = grp / Hkv;
  const int g = grp % Hkv;
  const int base = (b * Hq + g * G) * nqb;  // the group's items are contiguous
  const int count = G * nqb;
  auto bin_of = [&](int it) {
    const int c = min(max(cnt[base + it], 0), max_k);
    return kCostBins - 1 - min(c, kCostBins - 1);  // bin 0 = longest list
  };
  hist[tid] = 0;
  __syncthreads();
  for (int it = tid; it < count; it += kSchedThreads) atomicAdd(&hist[bin_of(it)], 1);
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  const int v = hist[tid];
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  hist[tid] = before + incl - v;  // exclusive offset of this bin
  __syncthreads();
  for (int it = tid; it < count; it += kSchedThreads) {
    const int rank = atomicAdd(&hist[bin_of(it)], 1);
    work[rank * ng + grp] = base + it;
  }
}

}  // namespace

hipError_t launch_schedule(const int32_t* cnt, int B, int Hq, int Hkv, int nqb, int max_k,
                           int32_t* work, hipStream_t stream) {
  if ((size_t)B * Hq * nqb == 0) return hipSuccess;
  hipLaunchKernelGGL(schedule_kernel, dim3(B * Hkv), dim3(kSchedThreads), 0, stream, cnt, Hq,
                     Hkv, nqb, max_k, work);
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
