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
// * A work item is one (batch, query head, query block).  Two wave64s serve an
//   item, wave w of the pair owning query rows 32w..32w+31.  The sparse pass
//   runs one item per workgroup.  The pooled pass runs two items of one KV
//   group per workgroup (HPW = 2 wave pairs): both read the same K/V, so each
//   K/V tile is copied to LDS once and used by both pairs (grouped-query
//   sharing of one K/V load), and the LDS per item halves.
// * Contractions use v_mfma_f32_32x32x16_bf16 in transposed form so that every
//   query row lives in one lane column:
//     S^T[kv][q] = K[kv][:] . Q[q][:]     (A = K tile from LDS, B = Q held in VGPRs)
//     O^T[d][q] += V^T[d][kv] . P^T[kv][q] (A = V^T tile from LDS, B = P^T straight
//                                          from the S^T accumulators)
//   Lane l then holds column q = l % 32 and half h = l / 32 of the rows, so a
//   row max or sum needs one cross-half exchange, and alpha and 1/l are
//   per-lane scalars.
// * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4, no
//   register staging).  Each wave-wide copy moves whole rows (coalesced 16-byte
//   lanes) into a padded slab, which keeps the fragment reads bank-conflict
//   free.  K fragments are plain 16-byte LDS reads; V^T fragments come from
//   ds_read_b64_tr_b16, which transposes 4x16 bf16 blocks on the fly into the
//   key order of P^T's registers.
// * K and V of a tile are separate pipeline stages.  The sparse pass streams
//   them in parts of 64 keys x 64 head-dims through a ring of three part slots
//   per workgroup (two parts in flight while one is computed on), and the small
//   footprint (26 KB) lets a CU hold 6 workgroups whose copies cover each
//   other's waits.  The pooled pass keeps a ring of two K slots and one V slot
//   per (two-item) workgroup, so K(j+1) streams in during tile j and V(j+1)
//   during QK of tile j+1.
// * exp2 with log2(e) folded into the softmax scale; fp32 row statistics; the
//   reference max is raised lazily (only when a tile exceeds it by 2^8), which
//   leaves O = acc / l unchanged and skips most accumulator rescales.
#include "seer_internal.h"

#include <math.h>

namespace seer {
namespace {

constexpr int kXcds = 8;        // MI355X: workgroups are dealt round-robin to 8 XCDs
constexpr int kPairThreads = 128;  // the two waves that serve one work item
// Two-item (four-wave) pooled workgroups one CU holds at once: 3 x 51 KB of
// LDS, and the kernel is held to 3 waves per SIMD (<= 168 VGPRs).
constexpr int kPairWgsPerCu = 3;
// The running row max is only raised when a tile's max exceeds it by more than
// this many powers of two; P values stay <= 2^8 and both O and l use the same
// reference max, so the result is unchanged while most tiles skip the rescale.
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct Cfg {
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per K/V row
  static constexpr int kRowsPerLoad = 64 / kChunks;      // rows per 1 KB wave-wide LDS load
  static constexpr int kLoadsPerTile = kBlk / kRowsPerLoad;
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

// The LDS-DMA reads M0 at issue, and gfx9 needs one wait state between an SALU
// write of M0 and an LDS-DMA instruction (the compiler's hazard pass cannot see
// inside the asm, so the s_nop is written here); M0 is declared clobbered.
__device__ __forceinline__ void dma16(uint64_t sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// Per-lane HBM byte offsets of this wave's share of one 64-row tile, the tile
// being copied by NW waves: slab n of wave w is slab w * NL + n; its lane L
// copies chunk L % chunks of row slab + S * (L / chunks).  Rows at or past
// `nvalid` (short last block) re-read the last valid row; those keys are always
// causally masked, and no LDS slot is left stale.
template <int D, int NW>
__device__ __forceinline__ void tile_offsets(uint32_t (&off)[Cfg<D>::kLoadsPerTile / NW],
                                             int nvalid, int wave, int lane) {
  constexpr int NL = Cfg<D>::kLoadsPerTile / NW;
  const int r = lane / Cfg<D>::kChunks;
  const int ch = lane % Cfg<D>::kChunks;
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int row = (wave * NL + n) + Cfg<D>::kLoadsPerTile * r;
    const int grow = row < nvalid ? row : nvalid - 1;
    off[n] = (uint32_t)((grow * D + ch * 8) * 2);
  }
}

// This wave's share (kLoadsPerTile / NW slabs) of every K or V tile copy.
template <int D, int NW>
struct TileIssue {
  static_assert(Cfg<D>::kKTileBytes <= Cfg<D>::kVTileBytes, "K fits the V slot");
  static_assert(Cfg<D>::kLoadsPerTile % NW == 0, "slabs split evenly over the waves");
  static constexpr int NL = Cfg<D>::kLoadsPerTile / NW;
  uint32_t off[NL];
  uint32_t kbase_lds, vbase_lds;  // LDS byte address of this wave's first slab
  __device__ __forceinline__ void init(const char* ks, const char* vs, int wave, int lane) {
    tile_offsets<D, NW>(off, kBlk, wave, lane);
    kbase_lds = lds_u32(ks) + wave * NL * Cfg<D>::kKSlab;
    vbase_lds = lds_u32(vs) + wave * NL * Cfg<D>::kVSlab;
  }
  // Issue this wave's share of a tile (K or V) whose first row is `g`.
  template <bool IS_V>
  __device__ __forceinline__ void issue(const __bf16* g, int nvalid, int wave, int lane,
                                        int slot_bytes) const {
    const uint64_t sb = uniform_u64(g);
    const uint32_t lb = (IS_V ? vbase_lds : kbase_lds) + slot_bytes;
    constexpr uint32_t stride = IS_V ? Cfg<D>::kVSlab : Cfg<D>::kKSlab;
    if (nvalid >= kBlk) {
#pragma unroll
      for (int n = 0; n < NL; ++n) dma16(sb, off[n], lb + n * stride);
    } else {
      // nvalid "redefined" here, so the clamped offsets cannot be computed
      // ahead of the branch: they stay off the common (full-tile) path.
      asm volatile("" : "+s"(nvalid));
      uint32_t o[NL];
      tile_offsets<D, NW>(o, nvalid, wave, lane);
#pragma unroll
      for (int n = 0; n < NL; ++n) dma16(sb, o[n], lb + n * stride);
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
// are requested before its MFMAs so the LDS latency is paid once.  `rw` is the
// wave's index within its pair (query rows 32 rw .. 32 rw + 31).
template <int D>
__device__ __forceinline__ void qk_tile(const RowState<D>& st, const char* ks, int lane, int rw,
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
    const int qrow = 32 * rw + col;
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

// This lane's value and that of lane ^ 32 (the other row half of the same
// query row), via v_permlane32_swap: one VALU op instead of an LDS permute.
struct HalfPair {
  float mine, other;
};
__device__ __forceinline__ HalfPair half_pair(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
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
  const HalfPair hp = half_pair(mx);
  mx = max3f(hp.mine, hp.other, -INFINITY);

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

// Q fragments of this wave's 32 rows (rows >= T read as zero) and a fresh state.
template <int D>
__device__ __forceinline__ void load_q(RowState<D>& st, const __bf16* __restrict__ qh, int q0,
                                       int T, int lane, int rw) {
  const int row = q0 + 32 * rw + (lane & 31);
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
                                         int T, int lane, int rw) {
  const HalfPair hl = half_pair(st.l);
  const float l = hl.mine + hl.other;
  const float inv = (l > 0.f) ? 1.0f / l : 0.f;
  const int row = q0 + 32 * rw + (lane & 31);
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
// Walk over the KV blocks of a pooled workgroup.  first() / next() return the
// next block in visiting order or -1 at the end; mine(j) tells a wave whether
// its own item uses block j.  All three are wave-uniform.

// Blocks 0..last in order; this wave's item uses blocks 0..own (own = -1 for
// an empty slot).
struct RangeWalk {
  int last, own, j;
  __device__ __forceinline__ int first() {
    j = 0;
    return last >= 0 ? 0 : -1;
  }
  __device__ __forceinline__ int next() { return ++j <= last ? j : -1; }
  __device__ __forceinline__ bool mine(int x) const { return x <= own; }
};

// The pooled pass's KV-block loop (a ring of K/V slots), run by all NW waves
// of the workgroup.  K tiles cycle through KS LDS slots and V tiles through VS slots;
// tile t's K lives in K slot t % KS and is replaced by K(t + KS) as soon as
// every wave has read it (after QK(t)), and likewise V(t + VS) replaces V(t)
// after PV(t).  With one slot each, K(t+1) streams in during softmax + PV of
// tile t and V(t+1) during QK of tile t+1; a second slot moves a copy one full
// tile earlier.  Every wave takes part in every copy and barrier; a wave
// computes on a tile only if walk.mine() says its item uses it, and then
// `on_tile(j, rowmax)` observes the tile.  `qi` is the item's query block (its
// diagonal tile).  The query fragments are loaded after the first tiles'
// copies are issued and everything is drained once before the loop, so Q's
// latency overlaps the first tiles' and the loop never waits on an older load.
//
// Waits: vmcnt counts this wave's copies in issue order, so "K(t) has landed"
// is "at most N copies issued after K(t) are outstanding", N being the copies
// the steady state issues after K(t): V(t) alone for KS = VS = 1, otherwise
// three tiles' worth (see the issue points above); likewise for V(t).  Near
// the end of the walk fewer copies follow, so there the loop drains to zero.
// (Tiles 0 and 1 need no special case: the prologue drained every copy.)
template <int D, int NW, int KS, int VS, bool EXACT_L, typename Walk, typename OnTile>
__device__ __forceinline__ void kv_loop(RowState<D>& st, const __bf16* __restrict__ qh, int q0,
                                        int qi, const __bf16* __restrict__ kh,
                                        const __bf16* __restrict__ vh, int T, Walk& walk,
                                        OnTile on_tile, char* ks, char* vs, int lane, int wave,
                                        int rw, float c) {
  constexpr int NL = Cfg<D>::kLoadsPerTile / NW;
  constexpr int M = KS > VS ? KS : VS;  // lookahead of the walk
  constexpr int kAfterK = (KS == 1 && VS == 1) ? NL : (KS == 1 ? NL : 3 * NL);
  constexpr int kAfterV = (KS == 1 && VS == 1) ? NL : (VS == 1 ? NL : 3 * NL);
  static_assert(KS >= 1 && KS <= 2 && VS >= 1 && VS <= 2, "one or two slots");
  // jq[m] = block of tile t + m (-1 past the end); jq[M] is fetched at the top
  // of each tile so that the walk's index loads overlap the tile's first wait.
  int jq[M + 1];
  jq[0] = walk.first();
  if (jq[0] < 0) {
    load_q<D>(st, qh, q0, T, lane, rw);
    return;
  }
#pragma unroll
  for (int m = 1; m < M; ++m) jq[m] = jq[m - 1] >= 0 ? walk.next() : -1;
  TileIssue<D, NW> io;
  io.init(ks, vs, wave, lane);
  auto issue_k = [&](int j, int slot) {
    io.template issue<false>(kh + (size_t)kBlk * j * D, T - kBlk * j, wave, lane,
                             slot * Cfg<D>::kKTileBytes);
  };
  auto issue_v = [&](int j, int slot) {
    io.template issue<true>(vh + (size_t)kBlk * j * D, T - kBlk * j, wave, lane,
                            slot * Cfg<D>::kVTileBytes);
  };
  issue_k(jq[0], 0);
  issue_v(jq[0], 0);
  if (KS == 2 && jq[1] >= 0) issue_k(jq[1], 1);  // KS or VS = 2 means M = 2
  if (VS == 2 && jq[1] >= 0) issue_v(jq[1], 1);
  load_q<D>(st, qh, q0, T, lane, rw);
  wait_vmcnt<0>();
  for (int t = 0;; ++t) {
    jq[M] = jq[M - 1] >= 0 ? walk.next() : -1;
    const int cur = jq[0];
    const bool own = walk.mine(cur);
    const int kslot = KS == 2 ? (t & 1) : 0;
    const int vslot = VS == 2 ? (t & 1) : 0;

    // K(t) has landed.  With one slot each, the only later copy is V(t), which
    // always exists; otherwise the copies after K(t) exist iff tile t+1 does.
    // (Deciding this without the newest lookahead keeps the walk's next index
    // load off the critical path.)
    if ((KS == 1 && VS == 1) || jq[1] >= 0) wait_vmcnt<kAfterK>(); else wait_vmcnt<0>();
    wg_barrier();
    f32x16 s[2];
    if (own) qk_tile<D>(st, ks + kslot * Cfg<D>::kKTileBytes, lane, rw, cur == qi, s);
    wg_barrier_reads_done();  // every wave is done reading K(t)
    if (jq[KS] >= 0) issue_k(jq[KS], kslot);
    if (own) {
      const float mx = softmax_tile<D, EXACT_L>(st, s, c);
      on_tile(cur, mx);
    }
    // V(t) has landed; the copies after it exist iff tile t + KS does.
    if (jq[KS] >= 0) wait_vmcnt<kAfterV>(); else wait_vmcnt<0>();
    wg_barrier();
    if (own) pv_tile<D, EXACT_L>(st, s, vs + vslot * Cfg<D>::kVTileBytes, lane);
    wg_barrier_reads_done();  // every wave is done reading V(t)
    if (jq[VS] >= 0) issue_v(jq[VS], vslot);
    if (jq[1] < 0) break;
#pragma unroll
    for (int m = 0; m < M; ++m) jq[m] = jq[m + 1];
  }
}

// ---------------------------------------------------------------------------
// Sparse prefill: one workgroup (one wave pair) per work-list entry, an entry
// being an item (b, h, i).
//
// Copies move in "parts": part p of a tile is its 64 keys x head-dims
// 64p..64p+63 of K or of V (8 KB; a D = 128 tile has two K parts and two V
// parts, a D = 64 tile one of each).  A tile is consumed part by part in the
// order K0 [K1] V0 [V1], and the parts of consecutive tiles form one stream
// that cycles through a ring of three LDS part slots: in step u (consuming
// stream part u) part u + 2 is requested into the slot part u - 1 vacated, so
// up to two parts are in flight while one is computed on.  One barrier per
// step serves both purposes: every wave has finished reading part u - 1 and
// has seen its own copies of part u land.  Three 8.5 KB slots let a CU hold 6
// workgroups (3 waves per SIMD, the VGPR limit).
//
// Within a step the copy is requested only after the step's LDS reads have
// been issued.  Requesting it first (copy, then LDS reads of another slot,
// with no s_waitcnt or barrier between them) returned corrupted K or V data
// now and then on MI355X: a few outputs per million moved by up to 0.004 and
// repeated runs differed.  With reads first, repeated runs are bit-identical
// (the GPU tests check this), and every other copy in this file is likewise
// separated from later LDS reads by a wait and a barrier.
//
// The contraction order is that of the whole-tile kernel (S^T accumulates
// k-steps 0..D/16-1 in order, O^T accumulates key steps 0..3 in order), so
// splitting a tile into parts does not change a single bit of the result.
//
// Pairing two heads of a KV group in one workgroup (as the pooled pass does)
// does not pay here: a pair walks the union of its two lists and the wave pair
// whose item skips a tile idles at the barriers.  On MI355X that loses 11 % at
// a union of 0.73 of the summed list lengths and wins 18 % only for identical
// dense lists (break-even near 0.62), while sparse rows of different heads
// overlap far less.
constexpr int kPartD = 64;                  // head-dims per part
constexpr int kPartRowBytes = 2 * kPartD;   // 128 B of one row in a part
constexpr int kPartSlabs = 8;               // 1 KB wave-wide copies per part
constexpr int kPartCopiesPerWave = kPartSlabs / 2;
// Slab n of a part holds rows n, n + 8, ..., n + 56 (each 128-byte row segment
// whole).  Slab strides keep the fragment reads conflict-free: K reads 16 rows
// at one 16-byte chunk (stride = 1 KB + 16 B: rows step by one 16-byte bank
// group), V transpose reads 4 rows x 64 B (stride = 1 KB + 64 B: rows step by
// 16 banks).  A slot fits either kind.
constexpr int kPartKSlab = 1024 + 16;
constexpr int kPartVSlab = 1024 + 64;
constexpr int kPartSlotBytes = kPartSlabs * kPartVSlab;
constexpr int kPartSlots = 3;

template <bool IS_V>
__device__ __forceinline__ int part_byte(int row, int chunk) {
  return (row % kPartSlabs) * (IS_V ? kPartVSlab : kPartKSlab) +
         (row / kPartSlabs) * kPartRowBytes + 16 * chunk;
}

// This wave's four copies of a part: copy n of wave w fills slab 4w + n; its
// lane L moves 16-byte chunk L % 8 of row (4w + n) + 8 (L / 8).  Rows at or
// past `nvalid` (short last block) re-read the last valid row; those keys are
// always causally masked.
template <int D>
struct PartIssue {
  uint32_t off[kPartCopiesPerWave];  // per-lane byte offset of a full tile's part 0
  uint32_t lds0;                     // LDS byte address of the ring
  int wave, lane;
  __device__ __forceinline__ void offsets(uint32_t (&o)[kPartCopiesPerWave], int nvalid) const {
#pragma unroll
    for (int n = 0; n < kPartCopiesPerWave; ++n) {
      const int row = (kPartCopiesPerWave * wave + n) + kPartSlabs * (lane >> 3);
      const int grow = row < nvalid ? row : nvalid - 1;
      o[n] = (uint32_t)((grow * D + (lane & 7) * 8) * 2);
    }
  }
  __device__ __forceinline__ void init(const char* ring, int w, int l) {
    wave = w;
    lane = l;
    offsets(off, kBlk);
    lds0 = lds_u32(ring);
  }
  // Copy part `p` of the K or V tile whose first row is `g` into the ring slot
  // starting `slot_off` bytes into the ring.
  template <bool IS_V>
  __device__ __forceinline__ void issue(const __bf16* g, int nvalid, int p, int slot_off) const {
    const uint64_t sb = uniform_u64(g + kPartD * p);
    constexpr uint32_t stride = IS_V ? kPartVSlab : kPartKSlab;
    const uint32_t lb = lds0 + slot_off + kPartCopiesPerWave * wave * stride;
    if (nvalid >= kBlk) {
#pragma unroll
      for (int n = 0; n < kPartCopiesPerWave; ++n) dma16(sb, off[n], lb + n * stride);
    } else {
      // nvalid "redefined" here, so the clamped offsets cannot be computed
      // ahead of the branch: they stay off the common (full-tile) path.
      asm volatile("" : "+s"(nvalid));
      uint32_t o[kPartCopiesPerWave];
      offsets(o, nvalid);
#pragma unroll
      for (int n = 0; n < kPartCopiesPerWave; ++n) dma16(sb, o[n], lb + n * stride);
    }
  }
};

// Step barrier: this wave's copies other than the newest N have landed and
// its LDS reads have returned; then every wave of the workgroup meets.
template <int N>
__device__ __forceinline__ void step_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// S^T += K_p Q_p^T for K part p (k-steps 4p..4p+3) of the tile in `ks`.
template <int D>
__device__ __forceinline__ void qk_part(const RowState<D>& st, const char* ks, int lane, int p,
                                        f32x16 (&s)[2]) {
  const int col = lane & 31;
  const int half = lane >> 5;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const char* krow = ks + part_byte<false>(32 * tt + col, half);
    bf16x8 kf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(krow + 32 * t);
    f32x16 a = p == 0 ? f32x16{} : s[tt];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], st.qf[4 * p + t], a, 0, 0, 0);
    s[tt] = a;
  }
}

__device__ __forceinline__ void mask_diag(f32x16 (&s)[2], int lane, int wave) {
  const int col = lane & 31;
  const int half = lane >> 5;
  const int qrow = 32 * wave + col;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kv = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
      if (kv > qrow) s[tt][r] = -INFINITY;
    }
}

// P^T as the bf16 B operands of the four 16-key steps, and its row sum (the
// sum of exactly the bf16 weights the MFMA uses) added to l.
template <int D>
__device__ __forceinline__ void p_operands(RowState<D>& st, const f32x16 (&s)[2],
                                           bf16x8 (&pb)[4]) {
  typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float lsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const f32x16& src = s[kk >> 1];
    const int o = 8 * (kk & 1);
    const f32x8 pv = {src[o + 0], src[o + 1], src[o + 2], src[o + 3],
                      src[o + 4], src[o + 5], src[o + 6], src[o + 7]};
    pb[kk] = __builtin_convertvector(pv, bf16x8);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16x2 pair = {pb[kk][2 * u], pb[kk][2 * u + 1]};
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lsum, false);
    }
  }
  st.l += lsum;
}

// O^T[d-tiles 2p, 2p+1] += V_p^T P^T for V part p of the tile in `vs`.
template <int D>
__device__ __forceinline__ void pv_part(RowState<D>& st, const bf16x8 (&pb)[4], const char* vs,
                                        int lane, int p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const int g = lane >> 4;
  const int i = lane & 15;
  const int h = g >> 1;
  const int r = i >> 2;
  const int sub = 4 * (i & 1);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int kv_a = 16 * kk + 4 * h + r;
    const int kv_b = kv_a + 8;
    const char* va_row = vs + part_byte<true>(kv_a, 2 * (g & 1) + ((i & 3) >> 1)) + 2 * sub;
    const char* vb_row = vs + part_byte<true>(kv_b, 2 * (g & 1) + ((i & 3) >> 1)) + 2 * sub;
    s16x4 va[2], vb[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      va[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(va_row + 64 * dt));
      vb[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vb_row + 64 * dt));
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const s16x8 vv = {va[dt][0], va[dt][1], va[dt][2], va[dt][3],
                        vb[dt][0], vb[dt][1], vb[dt][2], vb[dt][3]};
      st.acc[2 * p + dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, vv), pb[kk], st.acc[2 * p + dt], 0, 0, 0);
    }
  }
}

// An item's list as a walk over positions x = BS * entry + sub-tile (BS = list
// block size in 64-token tiles); position x stands for tile BS * list[x / BS] +
// x % BS and is usable when that entry lies in [0, ib] (ib = the item's own list
// row) and the tile does not pass the diagonal tile i.  The wave keeps 64
// consecutive positions in one VGPR (lane L: position base + L, its tile or -1)
// and their usable-mask from a ballot, so finding the next usable position is a
// find-first-set on scalar registers and reading its tile a v_readlane: no memory
// access on the tile loop's path except one window load per 64 positions.  The
// window load is an ordinary vector load; the compiler waits for it itself, and
// any copy issued before it is then waited for as well (never fewer).
template <int BS>
struct ListWindow {
  const int32_t* __restrict__ lst;
  int npos;  // BS * list length
  int ib, i;
  int base;  // first position of the window (a multiple of 64), -64 before the first load
  int win;
  uint64_t valid;
  // issue() requests the window starting at position b (lane L: list entry of
  // position b + L); finish() turns it into tiles and the usable-mask.  Split so
  // that other loads can be requested between the two.
  __device__ __forceinline__ void issue(int b, int lane) {
    base = b;
    const int x = b + lane;
    win = x < npos ? lst[x / BS] : -1;
  }
  __device__ __forceinline__ void finish(int lane) {
    const int x = base + lane;
    const int j = win;
    const int tile = BS * j + x % BS;
    const bool ok = x < npos && j >= 0 && j <= ib && tile <= i;
    win = ok ? tile : -1;
    valid = __builtin_amdgcn_ballot_w64(ok);
  }
  __device__ __forceinline__ void load(int b, int lane) {
    issue(b, lane);
    finish(lane);
  }
  // First usable position >= x, or npos if there is none.  Wave-uniform.
  __device__ __forceinline__ int next(int x, int lane) {
    while (x < npos) {
      if (x >= base + 64) load(x & ~63, lane);
      const uint64_t m = valid & (~0ull << (x - base));
      if (m != 0) return base + (int)__builtin_ctzll(m);
      x = base + 64;
    }
    return npos;
  }
  // Tile of usable position x (inside the current window).
  __device__ __forceinline__ int tile(int x) const {
    return __builtin_amdgcn_readlane(win, x - base);
  }
};

// The sparse pass's loop over one item's list (unusable positions are
// skipped, see ListWindow).  The last step reads its slot after the final
// barrier, so the ring must not be reused without another barrier (the kernel
// ends here).
template <int D, int BS>
__device__ __forceinline__ void kv_loop_parts(RowState<D>& st, const __bf16* __restrict__ qh,
                                              int q0, const __bf16* __restrict__ kh,
                                              const __bf16* __restrict__ vh, int T, int i,
                                              ListWindow<BS>& lw, int e, int j, char* ring,
                                              int lane, int wave, float c) {
  constexpr int NP = D / kPartD;           // K (and V) parts per tile
  constexpr int NL = kPartCopiesPerWave;   // this wave's copies per part
  // e = the first usable position, j = its tile (from the work entry).  The
  // first copies, the Q rows and the list window are all requested before the
  // one wait, so the item's start costs one memory latency.
  PartIssue<D> io;
  io.init(ring, wave, lane);
  // Stream parts 0 and 1: K0, K1 for D = 128; K, V for D = 64.
  io.template issue<false>(kh + (size_t)kBlk * j * D, T - kBlk * j, 0, 0);
  if (NP == 2)
    io.template issue<false>(kh + (size_t)kBlk * j * D, T - kBlk * j, 1, kPartSlotBytes);
  else
    io.template issue<true>(vh + (size_t)kBlk * j * D, T - kBlk * j, 0, kPartSlotBytes);
  load_q<D>(st, qh, q0, T, lane, wave);
  lw.issue(e & ~63, lane);
  wait_vmcnt<0>();
  lw.finish(lane);
  // Ring slots (byte offsets) of stream parts s, s + 1, s + 2 (mod 3), s being
  // the slot of the current tile's first part.  A tile of NP K and NP V parts
  // advances s by 2 NP = 1 (D = 128) or 2 (D = 64) modulo 3.
  int sa = 0, sb = kPartSlotBytes, sc = 2 * kPartSlotBytes;
  while (true) {
    const int cur = j;
    const __bf16* kc = kh + (size_t)kBlk * cur * D;
    const __bf16* vc = vh + (size_t)kBlk * cur * D;
    const int nc = T - kBlk * cur;
    bool more;
    f32x16 s[2];
    bf16x8 pb[4];
    if constexpr (NP == 2) {
      // Step K0: parts K0 (landing, slot a), K1 (slot b) in flight; request V0 (slot c).
      step_barrier<NL>();
      // The next usable entry is needed from step V0 on.
      e = lw.next(e + 1, lane);
      more = e < lw.npos;
      if (more) j = lw.tile(e);
      qk_part<D>(st, ring + sa, lane, 0, s);
      io.template issue<true>(vc, nc, 0, sc);
      // Step K1: K1 landing, V0 in flight; request V1 (slot a).
      step_barrier<NL>();
      qk_part<D>(st, ring + sb, lane, 1, s);
      io.template issue<true>(vc, nc, 1, sa);
      if (cur == i) {  // wave-uniform; the fence keeps it a branch
        compiler_fence();
        mask_diag(s, lane, wave);
      }
      (void)softmax_tile<D, false>(st, s, c);
      p_operands<D>(st, s, pb);
      const __bf16* kn = kh + (size_t)kBlk * j * D;
      const int nn = T - kBlk * j;
      // Step V0: V0 landing (slot c), V1 in flight; request K0 of the next tile (slot b).
      step_barrier<NL>();
      pv_part<D>(st, pb, ring + sc, lane, 0);
      if (more) io.template issue<false>(kn, nn, 0, sb);
      // Step V1: V1 landing (slot a), K0' in flight if any; request K1' (slot c).
      if (more) step_barrier<NL>(); else step_barrier<0>();
      pv_part<D>(st, pb, ring + sa, lane, 1);
      if (more) io.template issue<false>(kn, nn, 1, sc);
      const int t0 = sa;
      sa = sb;
      sb = sc;
      sc = t0;
    } else {
      e = lw.next(e + 1, lane);
      more = e < lw.npos;
      if (more) j = lw.tile(e);
      const __bf16* kn = kh + (size_t)kBlk * j * D;
      const __bf16* vn = vh + (size_t)kBlk * j * D;
      const int nn = T - kBlk * j;
      // Step K: K landing (slot a), V (slot b) in flight; request K of the next tile (slot c).
      step_barrier<NL>();
      qk_part<D>(st, ring + sa, lane, 0, s);
      if (more) io.template issue<false>(kn, nn, 0, sc);
      if (cur == i) {
        compiler_fence();
        mask_diag(s, lane, wave);
      }
      (void)softmax_tile<D, false>(st, s, c);
      p_operands<D>(st, s, pb);
      // Step V: V landing (slot b), K' in flight if any; request V' (slot a).
      if (more) step_barrier<NL>(); else step_barrier<0>();
      pv_part<D>(st, pb, ring + sb, lane, 0);
      if (more) io.template issue<true>(vn, nn, 0, sa);
      const int t0 = sc;
      sc = sb;
      sb = sa;
      sa = t0;
    }
    if (!more) break;
  }
}

// BS = list block size in 64-token tiles (1: 64-token blocks, 2: 128-token
// blocks).  Work items are always 64-row query blocks: item (b, h, i) reads
// list row i / BS, and each listed block j stands for the tiles BS j .. BS j +
// BS - 1, of which those past the diagonal tile i are skipped (a 128-token
// diagonal block is one full tile plus the masked diagonal tile for the second
// half of its rows, and the masked diagonal tile alone for the first half).
template <int D, int BS>
__global__ __launch_bounds__(kPairThreads, 3) void sparse_prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int Hq, int Hkv, int T, int nqb, float c, const int32_t* __restrict__ idx, int max_k,
    const int32_t* __restrict__ work, __bf16* __restrict__ o) {
  __shared__ __attribute__((aligned(1024))) char ring[kPartSlots * kPartSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int4 w4 = reinterpret_cast<const int4*>(work)[blockIdx.x];
  const int item = w4.x;
  if (item < 0) return;  // never written by the schedule (every rank holds an item)
  const int i = item % nqb;   // 64-row query block
  const int bh = item / nqb;  // b * Hq + h
  const int b = bh / Hq;
  const int g = (bh % Hq) / (Hq / Hkv);
  const size_t kv_off = ((size_t)b * Hkv + g) * (size_t)T * D;
  const size_t q_off = (size_t)bh * (size_t)T * D;

  RowState<D> st;
  const int rows = (nqb + BS - 1) / BS;  // list rows per head
  const int ib = i / BS;                 // this item's list row (and its own block)
  const size_t lrow = (size_t)bh * rows + ib;
  const int32_t* lst = idx + lrow * max_k;
  ListWindow<BS> lw{lst, BS * w4.w, ib, i, -64, -1, 0};
  if (w4.y < lw.npos) {
    kv_loop_parts<D, BS>(st, q + q_off, kBlk * i, k + kv_off, v + kv_off, T, i, lw, w4.y, w4.z,
                         ring, lane, wave, c);
  } else {  // no usable entry: O = 0
#pragma unroll
    for (int dt = 0; dt < Cfg<D>::kDTiles; ++dt) st.acc[dt] = f32x16{};
    st.l = 0.f;
  }
  (void)store_o<D>(st, o + q_off, kBlk * i, T, lane, wave);
}

// ---------------------------------------------------------------------------
// Pooled map: dense causal pass + per-tile row maxima, then the map rows.
//
// The items of KV group (b, g) are ordered by descending query block, then by
// head; workgroup L takes items HPW * p .. HPW * p + HPW - 1 of group
// L % (B * Hkv), with p = L / (B * Hkv).  So heavy rows start first; the items
// of a workgroup read the same K/V (same group) and sit at the same or at
// adjacent query blocks, so they share every tile but at most the last; and
// when the groups divide evenly over the 8 XCDs every workgroup of a group
// lands on the same XCD (workgroup L runs on XCD L % 8), keeping its K/V in
// that XCD's L2.
template <int D, int HPW, int KS, int VS>
__global__ __launch_bounds__(kPairThreads * HPW, kPairWgsPerCu) void pooled_map_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int B, int Hq, int Hkv, int T, int nqb, float c, __bf16* __restrict__ o,
    float* __restrict__ amap, float* __restrict__ rws) {
  constexpr int NT = kPairThreads * HPW;
  __shared__ __attribute__((aligned(1024))) char ks[KS * Cfg<D>::kKTileBytes];
  __shared__ __attribute__((aligned(1024))) char vs[VS * Cfg<D>::kVTileBytes];
  __shared__ float ms[HPW][kBlk];
  __shared__ float ils[HPW][kBlk];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave >> 1;
  const int rw = wave & 1;
  const int G = Hq / Hkv;
  const int ngroups = B * Hkv;
  const int p = blockIdx.x / ngroups;
  const int grp = blockIdx.x % ngroups;
  const int b = grp / Hkv;
  const int g = grp % Hkv;
  const long long per_group = (long long)G * nqb;
  int ii[HPW], hh[HPW];
  int last = -1;
#pragma unroll
  for (int x = 0; x < HPW; ++x) {
    const long long s = (long long)HPW * p + x;
    ii[x] = s < per_group ? nqb - 1 - (int)(s / G) : -1;  // -1: empty slot
    hh[x] = g * G + (s < per_group ? (int)(s % G) : 0);
    last = max(last, ii[x]);
  }
  const int i = ii[slot];
  const size_t bh = (size_t)b * Hq + hh[slot];
  const size_t kv_off = ((size_t)b * Hkv + g) * (size_t)T * D;
  const size_t q_off = bh * (size_t)T * D;
  const int q0 = i >= 0 ? kBlk * i : T;  // an empty slot has no rows below T
  // r_ij of a row block: packed lower triangle, 64 floats per tile.
  const size_t tri = (size_t)nqb * (nqb + 1) / 2;
  float* rrow = rws + (bh * tri + (size_t)max(i, 0) * (max(i, 0) + 1) / 2) * kBlk;

  RowState<D> st;
  RangeWalk walk{last, i, 0};
  auto on_tile = [&](int j, float mx) {
    if (lane < 32) rrow[(size_t)j * kBlk + 32 * rw + lane] = mx;
  };
  kv_loop<D, 2 * HPW, KS, VS, true>(st, q + q_off, q0, i, k + kv_off, v + kv_off, T, walk, on_tile, ks,
                            vs, lane, wave, rw, c);
  const float l = store_o<D>(st, o + q_off, q0, T, lane, rw);
  if (lane < 32) {
    const int r = 32 * rw + lane;
    const bool valid = q0 + r < T;
    ms[slot][r] = st.m;
    ils[slot][r] = (valid && l > 0.f) ? 1.0f / l : 0.f;  // rows past T take no part in the max
  }
  __syncthreads();

#pragma unroll
  for (int x = 0; x < HPW; ++x) {
    const int ix = ii[x];
    if (ix < 0) continue;
    const size_t bhx = (size_t)b * Hq + hh[x];
    const float* rx = rws + (bhx * tri + (size_t)ix * (ix + 1) / 2) * kBlk;
    float* arow = amap + (bhx * nqb + ix) * (size_t)nqb;
    for (int j = tid; j <= ix; j += NT) {
      const f32x4* rp = reinterpret_cast<const f32x4*>(rx + (size_t)j * kBlk);
      float a = 0.f;
#pragma unroll 4
      for (int r4 = 0; r4 < kBlk / 4; ++r4) {
        const f32x4 y = rp[r4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * r4 + u;
          a = fmaxf(a, __builtin_amdgcn_exp2f(fmaf(y[u], c, -ms[x][r])) * ils[x][r]);
        }
      }
      arow[j] = a;
    }
    for (int j = ix + 1 + tid; j < nqb; j += NT) arow[j] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Schedule (longest-processing-time first): one workgroup per KV group (b, g)
// counting-sorts that group's N = G * nQB items by descending list length.
// The groups run in P phases of GP = NG / P groups (NG = B * Hkv): the rank-r
// item of group q goes to position (q / GP) * GP * N + r * GP + q % GP of the
// work list.  Workgroups are dispatched in position order, so the groups of one
// phase run together, and within a phase long rows start first everywhere.
// Since the hardware deals workgroup L to XCD L % 8, every item of a group
// lands on the XCDs x with x % GP = q % GP whenever NG is a multiple of 8 (one
// XCD per group with one phase: its K/V then stays in that XCD's L2).  P > 1
// when the K and V of all groups exceed kActiveKvBytes: a phase's K/V then
// stays in the 256 MB memory-side cache while it runs, instead of every group's
// K/V competing for it (128k tokens, 8 KV groups: 64 MB per group, 8 phases).
constexpr int kSchedThreads = 1024;
constexpr int kCostBins = 1024;
constexpr double kActiveKvBytes = 64.0 * 1024 * 1024;

// Turns the histogram hist[kCostBins] into exclusive offsets (the first rank of
// each bin) in place and returns the total.  Called by the whole workgroup.
__device__ int bin_offsets(int* hist, int* wsum) {
  const int tid = threadIdx.x;
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
  int before = 0, total = 0;
  for (int w = 0; w < kSchedThreads / 64; ++w) {
    if (w < wv) before += wsum[w];
    total += wsum[w];
  }
  hist[tid] = before + incl - v;
  __syncthreads();
  return total;
}

// Items a schedule thread holds in registers: groups of up to 8192 items are
// sorted from one round of loads.
constexpr int kSchedIpt = 8;

// Each work entry is {item, first usable list position, its tile, list length}
// (an int4), so that the prefill workgroup can request its first K tile, its Q
// rows and its list window at once, with no chain of dependent loads.  An item
// without a usable position gets position = BS * length and tile -1.  The
// group's items are counting-sorted by descending cost (BS * length) in LDS.
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ idx, int Hq, int Hkv, int nqb,
    int bs, int max_k, int phases, int4* __restrict__ work) {
  __shared__ int hist[kCostBins];
  __shared__ int wsum[kSchedThreads / 64];
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int grp = blockIdx.x;
  const int ng = gridDim.x;
  const int bh0 = (grp / Hkv) * Hq + (grp % Hkv) * G;  // first head of the group
  const int base = bh0 * nqb;                          // the group's items
  const int rows = (nqb + bs - 1) / bs;                // list rows per head
  const int gp = ng / phases;                          // groups per phase
  const int ql = grp % gp;                             // the group's column in its phase
  const size_t pbase = (size_t)(grp / gp) * gp * G * nqb;  // first position of its phase
  const int N = G * nqb;
  auto row_of = [&](int it) { return (size_t)(bh0 + it / nqb) * rows + (it % nqb) / bs; };
  auto clamp_len = [&](int c) { return min(max(c, 0), max_k); };
  auto bin_of = [&](int n) { return kCostBins - 1 - min(bs * n, kCostBins - 1); };
  // The entry of item `it`, whose list holds n blocks and starts with j0 (the
  // first position is normally usable; otherwise the list is read on).
  auto entry = [&](int it, int n, int j0) -> int4 {
    const int32_t* lst = idx + row_of(it) * (size_t)max_k;
    const int i = it % nqb, ib = i / bs;
    int x = 0, tile = -1;
    for (; x < bs * n; ++x) {
      const int j = x < bs ? j0 : lst[x / bs];
      const int t = bs * j + x % bs;
      if (j >= 0 && j <= ib && t <= i) {
        tile = t;
        break;
      }
    }
    return {base + it, x, tile, n};
  };
  auto put = [&](int r, int4 e) { work[pbase + (size_t)r * gp + ql] = e; };
  hist[tid] = 0;
  __syncthreads();
  if (N <= kSchedIpt * kSchedThreads) {
    // Every count and first list entry of this thread's items requested at once
    // (indices clamped into the group, so no load sits behind a branch).
    int len[kSchedIpt], first[kSchedIpt];
#pragma unroll
    for (int u = 0; u < kSchedIpt; ++u) {
      const size_t row = row_of(min(tid + u * kSchedThreads, N - 1));
      len[u] = cnt[row];
      first[u] = idx[row * max_k];  // max_k >= 1
    }
#pragma unroll
    for (int u = 0; u < kSchedIpt; ++u) {
      len[u] = clamp_len(len[u]);
      if (tid + u * kSchedThreads < N) atomicAdd(&hist[bin_of(len[u])], 1);
    }
    __syncthreads();
    (void)bin_offsets(hist, wsum);
#pragma unroll
    for (int u = 0; u < kSchedIpt; ++u) {
      const int it = tid + u * kSchedThreads;
      if (it < N) put(atomicAdd(&hist[bin_of(len[u])], 1), entry(it, len[u], first[u]));
    }
  } else {
    for (int it = tid; it < N; it += kSchedThreads)
      atomicAdd(&hist[bin_of(clamp_len(cnt[row_of(it)]))], 1);
    __syncthreads();
    (void)bin_offsets(hist, wsum);
    for (int it = tid; it < N; it += kSchedThreads) {
      const size_t row = row_of(it);
      const int n = clamp_len(cnt[row]);
      put(atomicAdd(&hist[bin_of(n)], 1), entry(it, n, idx[row * max_k]));
    }
  }
}

constexpr float kLog2e = 1.4426950408889634f;
// K and V slots of the pooled kernel: a second K slot moves each K copy one
// tile earlier (+6 % measured; the sparse kernel's LDS leaves no room for it).
constexpr int kPairKSlots = 2;
constexpr int kPairVSlots = 1;


template <int D, int BS>
hipError_t sparse_launch(const void* q, const void* k, const void* v, size_t items, int Hq,
                         int Hkv, int T, int nqb, float c, const int32_t* idx, int max_k,
                         const int32_t* work, void* o, hipStream_t stream) {
  hipLaunchKernelGGL((sparse_prefill_kernel<D, BS>), dim3((unsigned)items), dim3(kPairThreads), 0,
                     stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, Hq, Hkv, T,
                     nqb, c, idx, max_k, work, (__bf16*)o);
  return hipGetLastError();
}

template <int D>
hipError_t pooled_launch(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                         int T, int nqb, float c, void* o, float* amap, float* rws,
                         hipStream_t stream) {
  constexpr int HPW = 2;
  const long long per_group = (long long)(Hq / Hkv) * nqb;
  const long long wgs = (long long)B * Hkv * ((per_group + HPW - 1) / HPW);
  hipLaunchKernelGGL((pooled_map_kernel<D, HPW, kPairKSlots, kPairVSlots>), dim3((unsigned)wgs), dim3(kPairThreads * HPW),
                     0, stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, B, Hq, Hkv,
                     T, nqb, c, (__bf16*)o, amap, rws);
  return hipGetLastError();
}

// Phases of the schedule for NG groups whose K and V take kv_bytes: the fewest
// (doubling from 1) that bring a phase's K/V to kActiveKvBytes, keeping each
// phase's groups an even share of the 8 XCDs (GP a multiple or a divisor of 8);
// 1 when NG is not a multiple of 8 (groups are not pinned to XCDs then).
int kv_phases(int ng, double kv_bytes) {
  int p = 1;
  if (ng % kXcds != 0) return p;
  while (kv_bytes / p > kActiveKvBytes && ng % (2 * p) == 0) {
    const int gp = ng / (2 * p);
    if (gp % kXcds != 0 && kXcds % gp != 0) break;
    p *= 2;
  }
  return p;
}

}  // namespace

// int32 entries: one int4 {item, first usable position, its tile, length} per item.
size_t sparse_work_entries(int B, int Hq, int, int nqb) { return (size_t)4 * B * Hq * nqb; }

hipError_t launch_sparse_prefill(const void* q, const void* k, const void* v, int B, int Hq,
                                 int Hkv, int T, int D, float sm_scale, int block,
                                 const int32_t* idx, const int32_t* cnt, int max_k, int32_t* work,
                                 void* o, hipStream_t stream) {
  const int nqb = (T + kBlk - 1) / kBlk;
  const size_t items = (size_t)B * Hq * nqb;
  if (items == 0) return hipSuccess;
  const float c = sm_scale * kLog2e;
  const int bs = block / kBlk;
  hipLaunchKernelGGL(schedule_kernel, dim3(B * Hkv), dim3(kSchedThreads), 0, stream, cnt, idx,
                     Hq, Hkv, nqb, bs, max_k, kv_phases(B * Hkv, 4.0 * B * Hkv * (double)T * D),
                     reinterpret_cast<int4*>(work));
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (bs == 2)
    return D == 128 ? sparse_launch<128, 2>(q, k, v, items, Hq, Hkv, T, nqb, c, idx, max_k,
                                            work, o, stream)
                    : sparse_launch<64, 2>(q, k, v, items, Hq, Hkv, T, nqb, c, idx, max_k,
                                           work, o, stream);
  return D == 128 ? sparse_launch<128, 1>(q, k, v, items, Hq, Hkv, T, nqb, c, idx, max_k,
                                          work, o, stream)
                  : sparse_launch<64, 1>(q, k, v, items, Hq, Hkv, T, nqb, c, idx, max_k, work,
                                         o, stream);
}

hipError_t launch_pooled_map(const void* q, const void* k, const void* v, int B, int Hq,
                             int Hkv, int T, int D, float sm_scale, void* o, float* amap,
                             float* rowmax_ws, hipStream_t stream) {
  const int nqb = (T + kBlk - 1) / kBlk;
  if ((size_t)B * Hq * nqb == 0) return hipSuccess;
  const float c = sm_scale * kLog2e;
  return D == 128 ? pooled_launch<128>(q, k, v, B, Hq, Hkv, T, nqb, c, o, amap, rowmax_ws, stream)
                  : pooled_launch<64>(q, k, v, B, Hq, Hkv, T, nqb, c, o, amap, rowmax_ws, stream);
}

}  // namespace seer
