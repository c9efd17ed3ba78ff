// AttnGate soft block scores: pooled Q and K, per-head linear layers, block
// RoPE and a causal softmax over the KV blocks.
//
// The gate pools along the sequence, Q by average and K by max and by min,
// concatenated along the hidden dimension before its linear layer (rebuttal
// "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs", Weakness
// 3 and "Question 1 (Theoretical or Intuitive Explanation for Pooling
// Selection)"), pools the Q and K from before the model's RoPE and adds its own
// block-level RoPE ("Q1 More about in AttnGate's RoPE"), and its output rows
// are a softmax ("Question 2: (Row-Normalization of Max-Pooled Attention
// Map)").  Threshold or TopK on these scores (seer_build_mask) gives the mask.
//
// Prefill kernels, up to 2048 query blocks (rows whose logits fit in LDS):
// * gate_pool_project_kernel: the pooling pass over K, K~ (linear layer and
//   block RoPE on the fp32 matrix cores) for every block, and the Q means of the
//   heavier half of the query groups.
// * gate_rows_kernel: per group of 16 query blocks, the Q pooling (lighter
//   half) or the means from the pass above, the linear layer and block RoPE, the
//   causal logits Q~ K~^T (fp32 matrix cores) into LDS, the exact row softmax,
//   the score rows written once; the fused variant selects each row's block list
//   from the same values.
// RoPE angles are formed and reduced in fp64 so that far block positions keep
// their accuracy.
// Longer rows (the logits go through HBM):
// * gate_pool_kernel: one wave per (batch, head, 64-token block) pools the block
//   (non-temporal 16-byte loads all in flight, lane shuffles to combine).
// * gate_project_kernel: one workgroup per (batch, head, 64 blocks) applies the
//   head's linear layer (v_mfma_f32_32x32x2f32) and the block RoPE.
// * gate_logits_kernel: one workgroup per causal 64 x 64 tile of block pairs
//   writes the scaled logits and each row's tile max and sum of exponentials;
//   gate_softmax_kernel then combines a row's partials in a fixed order and
//   normalises the row in place, zeros above the diagonal.
// * gate_softmax_mask_kernel: the same softmax straight into the row selection of
//   the mask build (mask_select.h); with a small workspace the logits are made
//   and selected in passes over tile rows.
// Decode kernels (one new token per sequence): gate_decode_pool_kernel and
// gate_project_kernel for the gate keys of every cache block,
// gate_decode_last_key_kernel for the block a token joins, gate_decode_scores_kernel
// and gate_decode_mask_kernel for the token's scores (and its block lists).
#include "mask_select.h"

#include <math.h>

namespace seer {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kTile = 64;  // query and key blocks per scores tile; tokens per block

// Pooling: one wave per (batch, head slot, 64-token block).  Lane L reads
// 16-byte chunk L % C of rows L / C, L / C + 64 / C, ... (C = D / 8 chunks per
// row), all its loads in flight at once; lanes holding the same chunk are
// combined with shuffles.  Q heads are averaged into pq [B, Hq, nQB, D], KV
// heads max- and min-pooled into pk [B, Hkv, nQB, 2D] ([max | min]).
constexpr int kPoolWaves = 8;

template <int D>
__global__ __launch_bounds__(64 * kPoolWaves) void gate_pool_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, int B, int Hq, int Hkv, int T,
    int nqb, float* __restrict__ pq, float* __restrict__ pk) {
  constexpr int C = D / 8;          // chunks per row
  constexpr int R = 64 / C;         // rows read together by the wave
  constexpr int kPerLane = kTile / R;
  const int lane = threadIdx.x & 63;
  // B (Hq + Hkv) nQB < 2^31 (checked by the host layer): 32-bit unit arithmetic.
  const int unit = blockIdx.x * kPoolWaves + (threadIdx.x >> 6);
  if (unit >= B * (Hq + Hkv) * nqb) return;
  const int i = unit % nqb;
  const int bh = unit / nqb;  // b * (Hq + Hkv) + head slot
  const int b = bh / (Hq + Hkv);
  const int slot = bh % (Hq + Hkv);
  const bool is_q = slot < Hq;
  const int head = is_q ? slot : slot - Hq;
  const int nheads = is_q ? Hq : Hkv;
  const __bf16* src = (is_q ? q : k) + ((size_t)b * nheads + head) * (size_t)T * D;
  const int ch = lane % C, rg = lane / C;
  const int r0 = kTile * i, r1 = min(r0 + kTile, T);
  bf16x8 x[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int r = r0 + rg + R * u;
    if (r < r1)  // read once: non-temporal, so it does not displace reused data in L2
      x[u] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8*>(src + (size_t)r * D + 8 * ch));
  }
  float a[8], m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = is_q ? 0.f : -INFINITY;
    m[e] = INFINITY;
  }
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    if (r0 + rg + R * u >= r1) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)x[u][e];
      if (is_q) {
        a[e] += v;
      } else {
        a[e] = fmaxf(a[e], v);
        m[e] = fminf(m[e], v);
      }
    }
  }
#pragma unroll
  for (int off = C; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ao = __shfl_xor(a[e], off, 64);
      const float mo = __shfl_xor(m[e], off, 64);
      a[e] = is_q ? a[e] + ao : fmaxf(a[e], ao);
      m[e] = fminf(m[e], mo);
    }
  if (rg == 0) {
    if (is_q) {
      float* out = pq + (((size_t)b * Hq + head) * nqb + i) * D + 8 * ch;
      const float inv = 1.0f / (float)(r1 - r0);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = a[e] * inv;
    } else {
      float* out = pk + (((size_t)b * Hkv + head) * nqb + i) * (2 * D) + 8 * ch;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        out[e] = a[e];
        out[D + e] = m[e];
      }
    }
  }
}

// Rotary pair (x1, x2) at block position pos with frequency inv_freq: the angle
// is formed and reduced mod 2 pi in fp64 (the multiple of 2 pi taken off is the
// nearest integer to the angle times 1 / (2 pi); near a half turn either
// neighbour leaves |r| <= pi + a few ulp, which sin and cos take as accurately),
// sin and cos of the reduced angle are fp32.
__device__ __forceinline__ void rope_rotate(double inv_freq, int pos, float x1, float x2,
                                            float& y1, float& y2) {
  const double two_pi = 6.283185307179586476925287;
  const double inv_two_pi = 0.159154943091895335768883763;
  const double ang = (double)pos * inv_freq;
  const float r = (float)(ang - two_pi * rint(ang * inv_two_pi));
  float sn, cs;
  sincosf(r, &sn, &cs);
  y1 = x1 * cs - x2 * sn;
  y2 = x2 * cs + x1 * sn;
}

// Rotary frequencies rope_base^(-2e/Dg), e < Dg/2, formed on the host in fp64
// and passed by value (a kernel argument): no per-lane pow on the device.
struct RopeFreqs {
  double f[64];
};

RopeFreqs rope_freqs(float rope_base, int dg) {
  RopeFreqs r{};
  for (int e = 0; e < dg / 2 && e < 64; ++e) r.f[e] = pow((double)rope_base, -2.0 * e / (double)dg);
  return r;
}

// Linear layer + block RoPE on the fp32 matrix cores.  One workgroup (two
// waves) per (batch, head slot, 64 pooled rows, column group); wave w computes
// rows 32 w .. 32 w + 31 of the group's 32-column tiles with
// v_mfma_f32_32x32x2f32, streaming 64-dim chunks of the rows and of the weights
// (stored transposed) through LDS, the next chunk's loads in flight during the
// current chunk's MFMAs.  In each group of 4 MFMAs a lane feeds 4 consecutive
// dims from one 16-byte read (lanes 0-31 and 32-63 take the two halves of an
// 8-dim group: any assignment of dims to MFMA k-slots works as long as both
// operands use the same one).  A column group is the tile pair {cg, cg + DG/64}
// that holds both columns e and e + DG/2 of a RoPE pair in the same lane; for
// DG = 32 the single tile holds the pair in lanes l and l ^ 16.  The block angle
// i * base^(-2e/DG) is formed and reduced mod 2 pi in fp64; sin and cos of the
// reduced angle are fp32.
constexpr int kProjWaves = 2;
constexpr int kProjTileRows = 32 * kProjWaves;  // pooled rows per workgroup
constexpr int kKChunk = 64;                     // input dims per LDS chunk

template <int DG>
struct ProjCfg {
  static constexpr int NT = DG / 32;               // 32-column tiles of the output
  static constexpr int NTW = NT >= 2 ? 2 : 1;      // tiles per workgroup
  static constexpr int NG = NT >= 2 ? NT / 2 : 1;  // column groups
};

template <int DG>
__global__ __launch_bounds__(64 * kProjWaves) void gate_project_kernel(
    const float* __restrict__ pq, const float* __restrict__ pk, int B, int Hq, int Hkv, int D,
    int nqb, const float* __restrict__ wq, const float* __restrict__ wk, float rope_base,
    float* __restrict__ qt, float* __restrict__ kt) {
  constexpr int NT = ProjCfg<DG>::NT;
  constexpr int NTW = ProjCfg<DG>::NTW;
  constexpr int NG = ProjCfg<DG>::NG;
  constexpr int NTH = 64 * kProjWaves;
  constexpr int WC = 32 * NTW;  // weight columns per workgroup
  __shared__ __attribute__((aligned(16))) float as[kProjTileRows][kKChunk + 4];
  __shared__ __attribute__((aligned(16))) float wt[WC][kKChunk + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int lr = lane & 31, hf = lane >> 5;
  const int ntiles = (nqb + kProjTileRows - 1) / kProjTileRows;
  const int cg = blockIdx.x % NG;
  const int tile = (blockIdx.x / NG) % ntiles;
  const int bh = blockIdx.x / NG / ntiles;
  const int b = bh / (Hq + Hkv);
  const int slot = bh % (Hq + Hkv);
  const bool is_q = slot < Hq;
  const int head = is_q ? slot : slot - Hq;
  const int nheads = is_q ? Hq : Hkv;
  const int din = is_q ? D : 2 * D;
  const float* a = (is_q ? pq : pk) + ((size_t)b * nheads + head) * nqb * din;
  const float* w = (is_q ? wq : wk) + (size_t)head * din * DG;
  const int i0 = kProjTileRows * tile;
  auto col0 = [&](int u) { return 32 * (cg + u * NG); };  // first column of tile u
  constexpr int kAVec = kProjTileRows * kKChunk / 4 / NTH;  // 16-byte row loads per thread
  constexpr int kWVec = kKChunk * WC / 4 / NTH;             // 16-byte weight loads per thread
  f32x4 va[kAVec], vw[kWVec];
  auto load = [&](int d0) {
#pragma unroll
    for (int n = 0; n < kAVec; ++n) {
      const int x = tid + NTH * n;
      const int r = x / (kKChunk / 4), c4 = x % (kKChunk / 4);
      va[n] = (i0 + r < nqb)
                  ? *reinterpret_cast<const f32x4*>(a + (size_t)(i0 + r) * din + d0 + 4 * c4)
                  : f32x4{};
    }
#pragma unroll
    for (int n = 0; n < kWVec; ++n) {
      const int x = tid + NTH * n;
      const int r = x / (WC / 4), c4 = x % (WC / 4);  // c4: 4-column group within WC
      const int col = col0(c4 / 8) + 4 * (c4 % 8);
      vw[n] = *reinterpret_cast<const f32x4*>(w + (size_t)(d0 + r) * DG + col);
    }
  };
  f32x16 acc[NTW];
#pragma unroll
  for (int u = 0; u < NTW; ++u) acc[u] = f32x16{};
  load(0);
  for (int d0 = 0; d0 < din; d0 += kKChunk) {
    __syncthreads();  // the previous chunk has been used
#pragma unroll
    for (int n = 0; n < kAVec; ++n) {
      const int x = tid + NTH * n;
      *reinterpret_cast<f32x4*>(&as[x / (kKChunk / 4)][4 * (x % (kKChunk / 4))]) = va[n];
    }
#pragma unroll
    for (int n = 0; n < kWVec; ++n) {
      const int x = tid + NTH * n;
      const int r = x / (WC / 4), c4 = x % (WC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) wt[4 * c4 + e][r] = vw[n][e];
    }
    __syncthreads();
    if (d0 + kKChunk < din) load(d0 + kKChunk);
#pragma unroll
    for (int g = 0; g < kKChunk / 8; ++g) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&as[32 * wv + lr][8 * g + 4 * hf]);
      f32x4 bv[NTW];
#pragma unroll
      for (int u = 0; u < NTW; ++u)
        bv[u] = *reinterpret_cast<const f32x4*>(&wt[32 * u + lr][8 * g + 4 * hf]);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
        for (int u = 0; u < NTW; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[k4], bv[u][k4], acc[u], 0, 0, 0);
    }
  }
  // acc[u][v]: row 32 wv + 8 (v / 4) + 4 hf + v % 4, column col0(u) + lr.
  float* out = (is_q ? qt : kt) + ((size_t)b * nheads + head) * nqb * DG;
  // Frequency of this lane's pair: e = col0(0) + lr, or lr % 16 for DG = 32.
  const int e_lane = NTW == 2 ? col0(0) + lr : (lr & 15);
  const double inv_freq = pow((double)rope_base, -2.0 * e_lane / (double)DG);
  auto rotate = [&](int i, float x1, float x2, float& y1, float& y2) {
    rope_rotate(inv_freq, i, x1, x2, y1, y2);
  };
  (void)NT;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = i0 + 32 * wv + 8 * (v / 4) + 4 * hf + (v % 4);
    if constexpr (NTW == 2) {
      const int e = col0(0) + lr;  // its partner e + DG/2 is column col0(1) + lr
      float y1, y2;
      rotate(i, acc[0][v], acc[1][v], y1, y2);
      if (i < nqb) {
        out[(size_t)i * DG + e] = y1;
        out[(size_t)i * DG + e + DG / 2] = y2;
      }
    } else {
      const float x = acc[0][v];
      const float xp = __shfl_xor(x, 16, 64);
      const bool low = lr < 16;  // column lr is e (low) or e + 16 (high) of its pair
      float y1, y2;
      rotate(i, low ? x : xp, low ? xp : x, y1, y2);
      if (i < nqb) out[(size_t)i * DG + lr] = low ? y1 : y2;
    }
  }
}

// Logits of one 64 x 64 tile of (query block, key block) pairs, tile (it, jt)
// with jt <= it, enumerated per head in row-major lower-triangular order, on
// the fp32 matrix cores: wave w computes the 32 x 32 quadrant (rows 32 (w / 2),
// columns 32 (w % 2)) with v_mfma_f32_32x32x2f32 from the two tiles in LDS
// (4 consecutive dims per lane and 16-byte read, as in the projection).  The
// tiles pass through LDS in two halves of the head dims, the second half's
// loads in flight during the first half's MFMAs (half the LDS: more
// workgroups per CU).
// Writes the scaled logits (-inf above the diagonal) and, per row, the tile's
// max and sum of exp(logit - max).  One launch covers the tile rows it0 ..
// it0 + (tile rows of npairs pairs) - 1; row i of head bh goes to row
// bh R + i - 64 it0 of `scores` (R rows per head: the whole map when R = nQB
// and it0 = 0, else one pass's rows), the pairs to the full-size `part`.
template <int DG>
__global__ __launch_bounds__(kScoreThreads) void gate_logits_kernel(
    const float* __restrict__ qt, const float* __restrict__ kt, int Hq, int Hkv, int nqb,
    float scale, int it0, int npairs, int R, float* __restrict__ scores,
    float2* __restrict__ part) {
  constexpr int DH = DG / 2;  // dims per half: the tiles go through LDS in two halves
  constexpr int kHalfTile = kTile * (DH + 4);
  constexpr int kSmem = 2 * kHalfTile > kTile * (kTile + 1) ? 2 * kHalfTile : kTile * (kTile + 1);
  // The Q and K half-tiles, later the 64 x 65 scaled logits.
  __shared__ __attribute__((aligned(16))) float smem[kSmem];
  float (*qs)[DH + 4] = reinterpret_cast<float (*)[DH + 4]>(smem);
  float (*ks)[DH + 4] = reinterpret_cast<float (*)[DH + 4]>(smem + kHalfTile);
  const int tid = threadIdx.x;
  const int ntiles = (nqb + kTile - 1) / kTile;
  const int pair = it0 * (it0 + 1) / 2 + (int)(blockIdx.x % npairs);
  const int bh = blockIdx.x / npairs;  // b * Hq + h
  int it = it0;
  while ((it + 1) * (it + 2) / 2 <= pair) ++it;
  const int jt = pair - it * (it + 1) / 2;
  const int b = bh / Hq;
  const int g = (bh % Hq) / (Hq / Hkv);
  const float* qrow = qt + (size_t)bh * nqb * DG;
  const float* krow = kt + ((size_t)b * Hkv + g) * nqb * DG;
  const int i0 = kTile * it, j0 = kTile * jt;
  constexpr int kVec = kTile * DH / 4 / kScoreThreads;  // 16-byte loads per thread and half
  f32x4 vq[kVec], vk[kVec];
  auto load = [&](int h) {
#pragma unroll
    for (int n = 0; n < kVec; ++n) {
      const int x = tid + kScoreThreads * n;
      const int r = x / (DH / 4), d4 = x % (DH / 4) + h * (DH / 4);
      vq[n] = (i0 + r < nqb) ? reinterpret_cast<const f32x4*>(qrow + (size_t)(i0 + r) * DG)[d4]
                             : f32x4{};
      vk[n] = (j0 + r < nqb) ? reinterpret_cast<const f32x4*>(krow + (size_t)(j0 + r) * DG)[d4]
                             : f32x4{};
    }
  };
  const int lane = tid & 63, wv = tid >> 6;
  const int lr = lane & 31, hf = lane >> 5;
  const int rb = 32 * (wv >> 1), cb = 32 * (wv & 1);
  f32x16 acc = {};
  load(0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h == 1) __syncthreads();  // every wave is done with the first half
#pragma unroll
    for (int n = 0; n < kVec; ++n) {
      const int x = tid + kScoreThreads * n;
      const int r = x / (DH / 4), d = 4 * (x % (DH / 4));
      *reinterpret_cast<f32x4*>(&qs[r][d]) = vq[n];
      *reinterpret_cast<f32x4*>(&ks[r][d]) = vk[n];
    }
    __syncthreads();
    if (h == 0) load(1);  // in flight during the first half's MFMAs
#pragma unroll 4
    for (int g8 = 0; g8 < DH / 8; ++g8) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&qs[rb + lr][8 * g8 + 4 * hf]);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&ks[cb + lr][8 * g8 + 4 * hf]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u], acc, 0, 0, 0);
    }
  }
  // acc[v]: tile row rb + 8 (v / 4) + 4 hf + v % 4, tile column cb + lr.  The
  // scaled, masked tile goes through LDS (over the Q tile) so that four threads
  // own each row: coalesced score rows and two-step row reductions.
  __syncthreads();  // every wave is done with qs and ks
  float (*st)[kTile + 1] = reinterpret_cast<float (*)[kTile + 1]>(smem);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = rb + 8 * (v / 4) + 4 * hf + (v % 4);
    const int i = i0 + r, j = j0 + cb + lr;
    st[r][cb + lr] = (i < nqb && j <= i) ? acc[v] * scale : -INFINITY;
  }
  __syncthreads();
  const int r = tid >> 2, qq = tid & 3;  // row r, columns 16 qq .. 16 qq + 15
  const int i = i0 + r;
  float x[16];
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    x[c] = st[r][16 * qq + c];
    mx = fmaxf(mx, x[c]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  float l = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int c = 0; c < 16; ++c) l += expf(x[c] - mx);  // exp(-inf) = 0 for masked entries
  }
  l += __shfl_xor(l, 1, 64);
  l += __shfl_xor(l, 2, 64);
  if (i < nqb) {
    float* srow = scores + ((size_t)bh * R + (i - kTile * it0)) * nqb + j0 + 16 * qq;
    if (j0 + 16 * qq + 16 <= nqb && (reinterpret_cast<uintptr_t>(srow) & 15) == 0) {
#pragma unroll
      for (int c = 0; c < 16; c += 4)
        *reinterpret_cast<f32x4*>(srow + c) = f32x4{x[c], x[c + 1], x[c + 2], x[c + 3]};
    } else {
      for (int c = 0; c < 16 && j0 + 16 * qq + c < nqb; ++c) srow[c] = x[c];
    }
    if (qq == 0) part[((size_t)bh * nqb + i) * ntiles + jt] = make_float2(mx, l);
  }
}

// One wave per score row: combine the row's per-tile (max, sum) pairs, then
// turn its logits into probabilities in place and zero the entries above the
// diagonal (including the tiles past the diagonal tile, never written above).
// The pairs (one per lane, 64 tiles at a time) and the row's first 512 entries
// are all requested before the combine; the combine reads the pairs lane by
// lane in tile order, so the result does not depend on timing.
constexpr int kRowWaves = 4;

// A row's (max, sum of exponentials) from its tiles' pairs pr[0 .. it], taken
// in tile order in every lane; `mine` holds pair `lane` (already requested).
__device__ __forceinline__ void combine_row_partials(const float2* __restrict__ pr, int it,
                                                     int lane, float2 mine, float& m, float& l) {
  m = -INFINITY;
  l = 0.f;
  for (int t0 = 0; t0 <= it; t0 += 64) {
    if (t0 > 0) mine = t0 + lane <= it ? pr[t0 + lane] : make_float2(-INFINITY, 0.f);
    const int tn = min(it - t0, 63);
    for (int t = 0; t <= tn; ++t) {
      const float px = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.x), t));
      const float py = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.y), t));
      if (px == -INFINITY) continue;
      const float mn = fmaxf(m, px);
      l = (m == -INFINITY ? 0.f : l * expf(m - mn)) + py * expf(px - mn);
      m = mn;
    }
  }
}

__global__ __launch_bounds__(64 * kRowWaves) void gate_softmax_kernel(
    int rows, int nqb, float* __restrict__ scores, const float2* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = row % nqb;
  const int ntiles = (nqb + kTile - 1) / kTile;
  const int it = i / kTile;
  const float2* pr = part + (size_t)row * ntiles;
  float* sr = scores + (size_t)row * nqb;
  // Causal part of the row in chunks of 512: entry j <= i, else a re-read of
  // entry i that is never used (no entry above the diagonal is read).
  constexpr int kPer = 8;
  float x[kPer];
  auto fetch = [&](int base) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) x[u] = sr[min(base + lane + 64 * u, i)];
  };
  float2 mine = lane <= it ? pr[lane] : make_float2(-INFINITY, 0.f);
  fetch(0);
  float m, l;
  combine_row_partials(pr, it, lane, mine, m, l);
  const float inv = 1.0f / l;
  for (int base = 0; base < nqb; base += 64 * kPer) {
    if (base > 0 && base <= i) fetch(base);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = base + lane + 64 * u;
      if (j < nqb) sr[j] = (j <= i) ? expf(x[u] - m) * inv : 0.f;
    }
  }
}

// Softmax and block selection of a score row in one pass (one wave per row,
// the whole causal row in registers, candidate j = 64 c + lane in slot c).
// The probabilities are those of gate_softmax_kernel, bit for bit, and the
// lists those seer_build_mask makes from them (same keys, same count rule,
// same select); with write_scores the probabilities also go back to the row.
// A launch takes the rows row0 .. row0 + Rv - 1 of every head (rows = B Hq Rv),
// their logits at row bh R + i - row0 of `logits` (R >= Rv rows per head).
template <int NPL>
__global__ __launch_bounds__(64 * kRowWaves) void gate_softmax_mask_kernel(
    int rows, int nqb, int row0, int Rv, int R, float* __restrict__ logits, int write_scores,
    const float2* __restrict__ part, int mode, float tau, double density, int keep_sink,
    int32_t* __restrict__ idx, int32_t* __restrict__ cnt, int max_k) {
  __shared__ int hist_all[kRowWaves][256];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int prow = blockIdx.x * kRowWaves + wv;  // row of this pass
  if (prow >= rows) return;
  const int bh = prow / Rv, il = prow % Rv;
  const int i = row0 + il;
  const int row = bh * nqb + i;  // B Hq nQB < 2^31 (checked by the host layer)
  const int n = i + 1;
  const int ntiles = (nqb + kTile - 1) / kTile;
  const int it = i / kTile;
  const float2* pr = part + (size_t)row * ntiles;
  float* sr = logits + ((size_t)bh * R + il) * nqb;
  float2 mine = lane <= it ? pr[lane] : make_float2(-INFINITY, 0.f);
  float x[NPL];
#pragma unroll
  for (int c = 0; c < NPL; ++c) x[c] = sr[min(64 * c + lane, i)];  // entries j > i unread
  float m, l;
  combine_row_partials(pr, it, lane, mine, m, l);
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    const int j = 64 * c + lane;
    x[c] = (j <= i) ? expf(x[c] - m) * inv : 0.f;
    if (write_scores && j < nqb) sr[j] = x[c];
  }
  uint32_t key[NPL];
  int npos = 0;
#pragma unroll
  for (int c = 0; c < NPL; ++c) {
    const int j = 64 * c + lane;
    uint32_t kj = 0u;
    if (j < n) {
      if (j == i || (keep_sink && j == 0))
        kj = 0xFFFFFFFFu;
      else
        kj = (mode == 1 || x[c] >= tau) ? rowsel::order_key(x[c]) : 0u;
    }
    key[c] = kj;
    npos += kj != 0u;
  }
  npos = rowsel::wave_sum(npos);
  int k;
  if (mode == 1) {
    const int forced = (i == 0) ? 1 : (keep_sink ? 2 : 1);
    k = min(i + 1, max(forced, (int)ceil(density * (double)(i + 1))));
  } else {
    k = min(npos, max_k);
  }
  const int count = rowsel::wave_select_row<NPL>(key, n, k, npos, lane, hist_all[wv],
                                                 idx + (size_t)row * max_k, max_k);
  if (lane == 0) cnt[row] = count;
}

// ---------------------------------------------------------------------------
// Prefill gate for nQB <= kRowsMaxBlocks: three kernels, the logits never leave
// the chip.
//
// gate_pool_project_kernel: the pooling pass over K and part of Q.  A K
// workgroup (first in the grid) takes 16 consecutive blocks of one KV head, 2
// per wave, pooled into LDS; then the 16 rows go through the head's linear
// layer on v_mfma_f32_16x16x4f32 (fp32 operands and accumulation) and the block
// RoPE: wave w computes RoPE tile pair w % P (16-column tiles holding columns e
// and e + Dg/2 in the same lane) over input-dim slice w / P, the slices summed
// in order through LDS.  At MFMA step s, lane group kg = lane / 16 feeds dim
// 16 (s / 4) + 4 kg + s % 4 of its row (one 16-byte LDS read per 4 steps) and
// the weight row of the same dim (any assignment of dims to k-slots works as
// long as both operands use it).  Q workgroups take 8 query blocks at or past
// qsplit (the heavier groups), one per wave, and write the means; the rest of Q
// is pooled by gate_rows_kernel, and all of it projected there.
constexpr int kPPWaves = 8;
constexpr int kPPRows = 16;   // pooled rows (blocks) per workgroup

// Pools block i of one head's rows src [T, D] into dst (Q: the D means; K: the
// D maxima then the D minima), its loads issued in SPLIT batches.  Lanes
// L < D / 8 write; a block at or past nqb gives zeros.  The sums run over the
// rows in the same order for any SPLIT.
template <int D, int SPLIT>
__device__ __forceinline__ void pool_block_lds(const __bf16* __restrict__ src, int T, int i,
                                               int nqb, bool is_q, int lane, float* dst) {
  constexpr int C = D / 8;   // chunks per row
  constexpr int R = 64 / C;  // rows read together by the wave
  constexpr int kPerLane = kTile / R;
  const int ch = lane % C, rg = lane / C;
  float a[8], m[8];
  if (i >= nqb) {
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dst[8 * ch + e] = 0.f;
        if (!is_q) dst[D + 8 * ch + e] = 0.f;
      }
    }
    return;
  }
  const int r0 = kTile * i, r1 = min(r0 + kTile, T);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = is_q ? 0.f : -INFINITY;
    m[e] = INFINITY;
  }
  // SPLIT batches of kPerLane / SPLIT loads, all of a batch in flight at once.
  constexpr int H = kPerLane / SPLIT;
#pragma unroll 1
  for (int h = 0; h < SPLIT; ++h) {
    bf16x8 x[H];
#pragma unroll
    for (int u = 0; u < H; ++u) {
      // Rows past a short last block re-read its last row (not used): the loads
      // stay unconditional, so none waits on another.  Read once: non-temporal,
      // so they do not displace reused data in L2.
      const int r = min(r0 + rg + R * (H * h + u), r1 - 1);
      x[u] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8*>(src + (size_t)r * D + 8 * ch));
    }
#pragma unroll
    for (int u = 0; u < H; ++u) {
      if (r0 + rg + R * (H * h + u) >= r1) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (float)x[u][e];
        if (is_q) {
          a[e] += v;
        } else {
          a[e] = fmaxf(a[e], v);
          m[e] = fminf(m[e], v);
        }
      }
    }
  }
#pragma unroll
  for (int off = C; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ao = __shfl_xor(a[e], off, 64);
      const float mo = __shfl_xor(m[e], off, 64);
      a[e] = is_q ? a[e] + ao : fmaxf(a[e], ao);
      m[e] = fminf(m[e], mo);
    }
  if (rg == 0) {
    if (is_q) {
      const float inv = 1.0f / (float)(r1 - r0);
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[8 * ch + e] = a[e] * inv;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dst[8 * ch + e] = a[e];
        dst[D + 8 * ch + e] = m[e];
      }
    }
  }
}

template <int D, int DG>
__global__ __launch_bounds__(64 * kPPWaves) __attribute__((amdgpu_waves_per_eu(6)))
void gate_pool_project_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, int B, int Hkv, int T, int nqb,
    int qsplit, const float* __restrict__ wk, RopeFreqs freqs, float* __restrict__ pq,
    float* __restrict__ kt) {
  constexpr int LDR = 2 * D + 4;  // padded LDS row (floats), room for a K row
  __shared__ __attribute__((aligned(16))) float prow[kPPRows][LDR];
  __shared__ float part[kPPWaves][2][4][64];  // each wave's share of the 16 x 2 x 16 products
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int ng = (nqb + kPPRows - 1) / kPPRows;
  const int kunits = B * Hkv * ng;
  if ((int)blockIdx.x >= kunits) {
    // Q: kPPWaves blocks at or past qsplit per workgroup, one per wave, means to pq.
    const int u = (int)blockIdx.x - kunits;
    const int nq8 = (nqb - qsplit + kPPWaves - 1) / kPPWaves;
    const int bh = u / nq8, i = qsplit + kPPWaves * (u % nq8) + wv;
    if (i < nqb)
      pool_block_lds<D, 2>(q + (size_t)bh * T * D, T, i, nqb, true, lane,
                           pq + ((size_t)bh * nqb + i) * D);
    return;
  }
  const int g = (int)blockIdx.x % ng, bh = (int)blockIdx.x / ng;  // bh = b * Hkv + head
  const int head = bh % Hkv;
  const int din = 2 * D;
  const __bf16* src = k + (size_t)bh * T * D;
#pragma unroll 1
  for (int t = 0; t < kPPRows / kPPWaves; ++t) {
    const int r = (kPPRows / kPPWaves) * wv + t;
    pool_block_lds<D, 2>(src, T, kPPRows * g + r, nqb, false, lane, &prow[r][0]);
  }
  __syncthreads();
  // Wave w: RoPE tile pair w % P (tiles w % P and w % P + Dg/32, columns e and
  // e + Dg/2), input dims of slice w / P of S (16-dim groups tb .. te - 1), the
  // weights of CB groups requested together.  The S slices' products are summed
  // in slice order through LDS.
  constexpr int P = DG / 32;
  constexpr int S = kPPWaves / P;
  constexpr int CB = 4;  // 16-dim groups whose weights are requested together
  const int pr = wv % P, ps = wv / P;
  const float* w = wk + (size_t)head * din * DG;
  const int r = lane & 15, kg = lane >> 4;
  const int col0 = 16 * pr + r, col1 = col0 + DG / 2;
  const int nt = din / 16;
  const int tb = ps * nt / S, te = (ps + 1) * nt / S;
  f32x4 acc0 = {}, acc1 = {};
  // Groups past the slice's end (a short last batch) re-read its last group
  // and enter with zero rows: straight-line loads, none waiting on another.
#pragma unroll 1
  for (int t0 = tb; t0 < te; t0 += CB) {
    float wr[CB][8];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int t = min(t0 + c, te - 1);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float* wrow = w + (size_t)(16 * t + 4 * kg + qq) * DG;
        wr[c][qq] = wrow[col0];
        wr[c][4 + qq] = wrow[col1];
      }
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int t = min(t0 + c, te - 1);
      f32x4 av = *reinterpret_cast<const f32x4*>(&prow[r][16 * t + 4 * kg]);
      if (t0 + c >= te) av = f32x4{};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[qq], wr[c][qq], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[qq], wr[c][4 + qq], acc1, 0, 0, 0);
      }
    }
  }
  // acc[v]: row 4 kg + v of the group, column col0 (acc0) or col1 (acc1).
  if constexpr (S > 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      part[wv][0][v][lane] = acc0[v];
      part[wv][1][v][lane] = acc1[v];
    }
    __syncthreads();
    if (ps != 0) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      acc0[v] = part[pr][0][v][lane];
      acc1[v] = part[pr][1][v][lane];
    }
#pragma unroll 1
    for (int s2 = 1; s2 < S; ++s2)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc0[v] += part[pr + P * s2][0][v][lane];
        acc1[v] += part[pr + P * s2][1][v][lane];
      }
  }
  float* out = kt + (size_t)bh * nqb * DG;
  const double inv_freq = freqs.f[col0];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int i = kPPRows * g + 4 * kg + v;
    float y1, y2;
    rope_rotate(inv_freq, i, acc0[v], acc1[v], y1, y2);
    if (i < nqb) {
      out[(size_t)i * DG + col0] = y1;
      out[(size_t)i * DG + col1] = y2;
    }
  }
}

// gate_rows_kernel: the Q~ rows, logits, softmax (and with MASK the block
// selection) of one group of 16 query blocks of one (batch, head).  Group g has
// g + 1 tiles of 16 x 16 logits.  Workgroups take the groups in blocks of 8
// weight ranks, heaviest block first, alternately heaviest-first and
// lightest-first within a block, so that the workgroups resident together on a
// CU (dealt out in launch order) carry about equal work, and one group's softmax
// overlaps another's matrix work.  Only the logits take LDS and the registers
// stay within 128, so four workgroups fit on a CU at 512 query blocks (all of
// them at once for 32 heads).
// * Q~ rows: the group's 16 query blocks are pooled (means) into LDS (or, for the
//   heavier groups, their means are copied from gate_pool_project_kernel), go through
//   the head's linear layer on v_mfma_f32_16x16x4f32 (wave w < Dg/32 takes RoPE
//   tile pair w, columns e and e + Dg/2, over all D input dims, dims assigned to
//   k-slots as in gate_pool_project_kernel) and the block RoPE, and each lane then
//   holds its Q~ operands in registers.
// * Logits: the waves take the tiles round robin, Q~ K~^T on
//   v_mfma_f32_16x16x4f32 (the next tile's K~ rows loading during the current
//   tile's MFMAs), and write the scaled logits (-inf above the diagonal) into
//   LDS.
// * Softmax: one wave per row takes the exact row max, the sum of exponentials
//   and the probabilities in registers; the score row is written once (zeros
//   above the diagonal) and, with MASK, selected as in gate_softmax_mask_kernel
//   (same keys, count rule and select).  Both variants share the softmax code,
//   so the fused lists are those of the scores, bit for bit.
constexpr int kRowGroup = 16;         // query blocks per row group
constexpr int kRowsWaves = 4;
constexpr int kRowsMaxBlocks = 2048;
constexpr int kGateSplitNum = 1, kGateSplitDen = 2;  // share of groups pooled in the rows kernel  // LDS: 16 nQB fp32 logits per workgroup

// Wave-wide max and sum with the same value in every lane.  Within each row of
// 16 lanes, DPP moves pair every lane with a partner holding the same partial
// (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror): both add the
// same two operands, in either order, which is exact for a commutative
// operation.  The four row results are then combined in one fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_lanes(float v, int r) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
}

__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(row_lanes(v, 0), row_lanes(v, 1)), fmaxf(row_lanes(v, 2), row_lanes(v, 3)));
}

__device__ __forceinline__ float wave_sum_f(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (row_lanes(v, 0) + row_lanes(v, 1)) + (row_lanes(v, 2) + row_lanes(v, 3));
}

// Dynamic LDS of gate_rows_kernel: first the pooled Q rows [16][D + 4] and the
// Q~ rows [16][Dg + 4], then, in the same space, the logits of the group
// (16 x 16 G fp32).
size_t gate_rows_lds_bytes(int nqb, int d, int dg) {
  const int G = (nqb + kRowGroup - 1) / kRowGroup;
  const size_t logits = (size_t)kRowGroup * kRowGroup * G;
  const size_t qrows = (size_t)kRowGroup * (d + 4) + (size_t)kRowGroup * (dg + 4);
  return (logits > qrows ? logits : qrows) * sizeof(float);
}

template <int D, int DG, int NPL, bool MASK>
__global__ __launch_bounds__(64 * kRowsWaves) __attribute__((amdgpu_waves_per_eu(4))) void gate_rows_kernel(
    const __bf16* __restrict__ q, int T, const float* __restrict__ pq, int qsplit,
    const float* __restrict__ wq, RopeFreqs freqs,
    const float* __restrict__ kt, int BHq, int Hq, int Hkv, int nqb, float scale,
    float* __restrict__ scores, int mode, float tau, double density, int keep_sink,
    int32_t* __restrict__ idx, int32_t* __restrict__ cnt, int max_k) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int hist_all[MASK ? kRowsWaves : 1][256];
  constexpr int NV = DG / 16;     // 16-byte operand reads per lane and row
  float* lg = smem;  // logits [16][16 (g + 1)], once the Q~ operands are in registers
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15, kg = lane >> 4;
  const int G = (nqb + kRowGroup - 1) / kRowGroup;
  const int bh = (int)(blockIdx.x % BHq);  // b * Hq + h
  int g;
  {
    const int j = (int)(blockIdx.x / BHq);  // weight rank: 0 is the heaviest group
    const int lo = j / 8 * 8, hi = min(G, lo + 8);
    const int jj = ((j / 8) & 1) ? hi - 1 - (j - lo) : j;
    g = G - 1 - jj;
  }
  const int b = bh / Hq;
  const int kvh = b * Hkv + (bh % Hq) / (Hq / Hkv);
  const int ntile = g + 1;
  const int width = kRowGroup * ntile;  // logit row length in LDS

  // Q~ of the group: pooled means (blocks past nQB give zero rows, whose logits
  // are never read), the linear layer and the block RoPE, into LDS.
  constexpr int LDQ = D + 4, LDT = DG + 4;  // padded LDS rows (floats)
  float* prow = smem;                 // pooled Q means [16][LDQ]
  float* qs = smem + kRowGroup * LDQ;  // Q~ rows [16][LDT]
  if (kRowGroup * g >= qsplit) {
    // Pooled by gate_pool_project_kernel: copy the means.
    constexpr int C4 = D / 4;
    for (int x = threadIdx.x; x < kRowGroup * C4; x += 64 * kRowsWaves) {
      const int rr = x / C4, i = min(kRowGroup * g + rr, nqb - 1);
      f32x4 v = *reinterpret_cast<const f32x4*>(pq + ((size_t)bh * nqb + i) * D + 4 * (x % C4));
      if (kRowGroup * g + rr >= nqb) v = f32x4{};
      *reinterpret_cast<f32x4*>(prow + rr * LDQ + 4 * (x % C4)) = v;
    }
  } else {
#pragma unroll 1
    for (int t = 0; t < kRowGroup / kRowsWaves; ++t) {
      const int rr = (kRowGroup / kRowsWaves) * wv + t;
      pool_block_lds<D, 1>(q + (size_t)bh * T * D, T, kRowGroup * g + rr, nqb, true, lane,
                           prow + rr * LDQ);
    }
  }
  __syncthreads();
  if (wv < DG / 32) {
    // RoPE tile pair wv: columns col0 and col0 + Dg/2, all D input dims, the
    // weights of CB 16-dim groups requested together.
    constexpr int NT = D / 16;
    constexpr int CB = 4;
    const float* w = wq + (size_t)(bh % Hq) * D * DG;
    const int col0 = 16 * wv + r, col1 = col0 + DG / 2;
    f32x4 acc0 = {}, acc1 = {};
#pragma unroll 1
    for (int t0 = 0; t0 < NT; t0 += CB) {
      float wr[CB][8];
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int t = min(t0 + c, NT - 1);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float* wrow = w + (size_t)(16 * t + 4 * kg + qq) * DG;
          wr[c][qq] = wrow[col0];
          wr[c][4 + qq] = wrow[col1];
        }
      }
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int t = min(t0 + c, NT - 1);
        f32x4 av = *reinterpret_cast<const f32x4*>(prow + r * LDQ + 16 * t + 4 * kg);
        if (t0 + c >= NT) av = f32x4{};
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[qq], wr[c][qq], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[qq], wr[c][4 + qq], acc1, 0, 0, 0);
        }
      }
    }
    // acc[v]: row 4 kg + v of the group, column col0 (acc0) or col1 (acc1).
    const double inv_freq = freqs.f[col0];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float y1, y2;
      rope_rotate(inv_freq, kRowGroup * g + 4 * kg + v, acc0[v], acc1[v], y1, y2);
      qs[(4 * kg + v) * LDT + col0] = y1;
      qs[(4 * kg + v) * LDT + col1] = y2;
    }
  }
  __syncthreads();
  // This lane's Q~ operands (row r of the group, dims 16 t + 4 kg .. + 3), held in
  // registers for every tile.
  f32x4 qv[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t)
    qv[t] = *reinterpret_cast<const f32x4*>(qs + r * LDT + 16 * t + 4 * kg);
  __syncthreads();  // the logits below reuse this LDS

  // Logits: lane (r, kg) feeds dims 16 t + 4 kg .. + 3 of row r of both
  // operands at MFMA steps 4 t .. 4 t + 3.  K~ rows past nQB (the last group's
  // diagonal tile) re-read the last row: those logits are all above the
  // diagonal, and the loads stay unconditional.
  const float* krow = kt + (size_t)kvh * nqb * DG + 4 * kg;
  auto load_k = [&](int ct, f32x4 (&v)[NV]) {
    const float* src = krow + (size_t)min(kRowGroup * ct + r, nqb - 1) * DG;
#pragma unroll
    for (int t = 0; t < NV; ++t) v[t] = *reinterpret_cast<const f32x4*>(src + 16 * t);
  };
  auto tile = [&](int ct, const f32x4 (&bk)[NV]) {
    f32x4 acc = {};
#pragma unroll
    for (int t = 0; t < NV; ++t) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qv[t][qq], bk[t][qq], acc, 0, 0, 0);
    }
    // acc[v]: row 4 kg + v of the group, column 16 ct + r.
    const int j = kRowGroup * ct + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int lr = 4 * kg + v;
      lg[lr * width + j] = (j <= kRowGroup * g + lr) ? acc[v] * scale : -INFINITY;
    }
  };
  // Tiles in pairs with two buffers: no branch between a prefetch and its use
  // (one would let the compiler sink the load to the use), and the scheduling
  // barriers keep the loads ahead of the MFMAs they overlap.  A tile index past
  // the last re-reads the last tile's rows, so every wait counts exactly the
  // loads of the tile after it.
  f32x4 b0[NV], b1[NV];
  int ct = wv;
  load_k(min(ct, ntile - 1), b0);
#pragma unroll 1
  for (; ct + kRowsWaves < ntile; ct += 2 * kRowsWaves) {
    load_k(ct + kRowsWaves, b1);
    __builtin_amdgcn_sched_barrier(0);
    tile(ct, b0);
    load_k(min(ct + 2 * kRowsWaves, ntile - 1), b0);
    __builtin_amdgcn_sched_barrier(0);
    tile(ct + kRowsWaves, b1);
  }
  if (ct < ntile) tile(ct, b0);
  __syncthreads();

#pragma unroll 1
  for (int lr = wv; lr < kRowGroup; lr += kRowsWaves) {
    const int i = kRowGroup * g + lr;
    if (i >= nqb) break;
    const float* src = lg + lr * width;
    float x[NPL];
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NPL; ++c) {
      const int j = 64 * c + lane;
      x[c] = j <= i ? src[j] : -INFINITY;
      m = fmaxf(m, x[c]);
    }
    m = wave_max_f(m);
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < NPL; ++c) {
      x[c] = (64 * c + lane <= i) ? expf(x[c] - m) : 0.f;
      l += x[c];
    }
    l = wave_sum_f(l);
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < NPL; ++c) x[c] *= inv;
    const size_t row = (size_t)bh * nqb + i;
    if (scores) {
      // Written once, read by the caller later: non-temporal, so the stream of
      // score rows does not push the K~ rows out of L2.
      float* sr = scores + row * nqb;
#pragma unroll
      for (int c = 0; c < NPL; ++c)
        if (64 * c + lane < nqb) __builtin_nontemporal_store(x[c], sr + 64 * c + lane);
    }
    if constexpr (MASK) {
      const int n = i + 1;
      uint32_t key[NPL];
      int npos = 0;
#pragma unroll
      for (int c = 0; c < NPL; ++c) {
        const int j = 64 * c + lane;
        uint32_t kj = 0u;
        if (j < n) {
          if (j == i || (keep_sink && j == 0))
            kj = 0xFFFFFFFFu;
          else
            kj = (mode == 1 || x[c] >= tau) ? rowsel::order_key(x[c]) : 0u;
        }
        key[c] = kj;
        npos += kj != 0u;
      }
      npos = rowsel::wave_sum(npos);
      int kk;
      if (mode == 1) {
        const int forced = (i == 0) ? 1 : (keep_sink ? 2 : 1);
        kk = min(i + 1, max(forced, (int)ceil(density * (double)(i + 1))));
      } else {
        kk = min(npos, max_k);
      }
      const int count = rowsel::wave_select_row<NPL>(key, n, kk, npos, lane, hist_all[wv],
                                                     idx + row * max_k, max_k);
      if (lane == 0) cnt[row] = count;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-token gate of decoding (no query pooling).  Gate keys: K is pooled per block
// of the cache exactly as above but up to each sequence's own length, and the
// pooled rows go through gate_project_kernel (K slots only) -- or, to refresh
// only each sequence's last block (the one a new token joins), one row per
// (sequence, KV head) through gate_decode_last_key_kernel.  Scores: the token's q
// through the Q layer and the rotation at its block index nb - 1, then one
// workgroup per (sequence, query head) takes the logits over the sequence's
// blocks and their softmax.

// One wave per (sequence, KV head, block): [max | min] over the block's tokens
// below kv_len, in 64-row steps (non-temporal loads, lane shuffles to combine).
// Blocks at or past the end of the sequence are not written.
template <int D>
__global__ __launch_bounds__(64 * kPoolWaves) void gate_decode_pool_kernel(
    const __bf16* __restrict__ k, const int32_t* __restrict__ kv_len, int B, int Hkv, int Tmax,
    int nkb, int bs, float* __restrict__ pk) {
  constexpr int C = D / 8;   // chunks per row
  constexpr int R = 64 / C;  // rows read together by the wave
  constexpr int kPerLane = kTile / R;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * kPoolWaves + (threadIdx.x >> 6);
  if (unit >= B * Hkv * nkb) return;
  const int bg = unit / nkb;
  const int len = min(max(kv_len[bg / Hkv], 0), Tmax);
  const int j = unit % nkb;
  const int r0 = bs * j, r1 = min(r0 + bs, len);
  if (r0 >= r1) return;
  const __bf16* src = k + (size_t)bg * Tmax * D;
  const int ch = lane % C, rg = lane / C;
  float a[8], m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = -INFINITY;
    m[e] = INFINITY;
  }
  for (int s0 = r0; s0 < r1; s0 += kTile) {
    bf16x8 x[kPerLane];
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      const int r = s0 + rg + R * u;
      if (r < r1)
        x[u] = __builtin_nontemporal_load(
            reinterpret_cast<const bf16x8*>(src + (size_t)r * D + 8 * ch));
    }
#pragma unroll
    for (int u = 0; u < kPerLane; ++u) {
      if (s0 + rg + R * u >= r1) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (float)x[u][e];
        a[e] = fmaxf(a[e], v);
        m[e] = fminf(m[e], v);
      }
    }
  }
#pragma unroll
  for (int off = C; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = fmaxf(a[e], __shfl_xor(a[e], off, 64));
      m[e] = fminf(m[e], __shfl_xor(m[e], off, 64));
    }
  if (rg == 0) {
    float* out = pk + ((size_t)bg * nkb + j) * (2 * D) + 8 * ch;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      out[e] = a[e];
      out[D + e] = m[e];
    }
  }
}

// Projection of one staged gate row on the VALU by a 256-thread workgroup: xs
// (LDS, din <= 256 inputs) times W [din, DG]; wave w sums input dims
// [w din/4, (w+1) din/4) for columns t and t + DG/2 (lane t < DG/2), 16 weight
// pairs in flight at a time; wave 0 adds the four partial sums in order,
// rotates the pair at block position pos and stores y[t], y[t + DG/2] (y may be
// in LDS or global memory).  Called by the whole workgroup; ends with a barrier.
constexpr int kRowThreads = 256;

template <int DG>
__device__ __forceinline__ void project_row(const float* xs, int din, const float* __restrict__ wr,
                                            float (*part)[2][DG / 2], int pos, float rope_base,
                                            float* y) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = din / (kRowThreads / 64);  // din is 64, 128 or 256
  const int d0 = wv * per;
  if (lane < DG / 2) {
    float x1 = 0.f, x2 = 0.f;
    for (int dd = 0; dd < per; dd += 16) {
      float w1[16], w2[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const size_t o = (size_t)(d0 + dd + u) * DG + lane;
        w1[u] = wr[o];
        w2[u] = wr[o + DG / 2];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        x1 = fmaf(xs[d0 + dd + u], w1[u], x1);
        x2 = fmaf(xs[d0 + dd + u], w2[u], x2);
      }
    }
    part[wv][0][lane] = x1;
    part[wv][1][lane] = x2;
  }
  __syncthreads();
  if (wv == 0 && lane < DG / 2) {
    const float x1 = ((part[0][0][lane] + part[1][0][lane]) + part[2][0][lane]) + part[3][0][lane];
    const float x2 = ((part[0][1][lane] + part[1][1][lane]) + part[2][1][lane]) + part[3][1][lane];
    const double inv_freq = pow((double)rope_base, -2.0 * lane / (double)DG);
    float y1, y2;
    rope_rotate(inv_freq, pos, x1, x2, y1, y2);
    y[lane] = y1;
    y[lane + DG / 2] = y2;
  }
  __syncthreads();
}

// Gate key of each sequence's last block, one 256-thread workgroup per
// (sequence, KV head): the block's tokens below kv_len are max- and min-pooled
// (16 rows x 16 chunks of 8 dims per pass, non-temporal 16-byte loads, the 16
// row groups then combined in LDS), and the pooled row [max | min] is projected
// with Wk[g] and rotated at the block index, into k_gate.
template <int D, int DG>
__global__ __launch_bounds__(kRowThreads) void gate_decode_last_key_kernel(
    const __bf16* __restrict__ k, const int32_t* __restrict__ kv_len, int Hkv, int Tmax, int nkb,
    int bs, const float* __restrict__ wk, float rope_base, float* __restrict__ kt) {
  constexpr int C = D / 8;                 // 16-byte chunks per row
  constexpr int RG = kRowThreads / C;      // row groups per pass
  __shared__ float gmax[RG][D], gmin[RG][D];
  __shared__ float xs[2 * D];
  __shared__ float part[kRowThreads / 64][2][DG / 2];
  const int bg = blockIdx.x;
  const int tid = threadIdx.x;
  const int len = min(max(kv_len[bg / Hkv], 0), Tmax);
  if (len == 0) return;  // the whole workgroup leaves together
  const int j = (len - 1) / bs;
  const int r0 = bs * j, r1 = len;
  const __bf16* src = k + (size_t)bg * Tmax * D;
  const int ch = tid % C, rg = tid / C;
  float a[8], m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = -INFINITY;
    m[e] = INFINITY;
  }
  constexpr int kMaxPass = 128 / RG;  // bs <= 128
  bf16x8 xv[kMaxPass];
#pragma unroll
  for (int u = 0; u < kMaxPass; ++u) {
    const int r = r0 + rg + RG * u;
    if (r < r1)
      xv[u] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8*>(src + (size_t)r * D + 8 * ch));
  }
#pragma unroll
  for (int u = 0; u < kMaxPass; ++u) {
    if (r0 + rg + RG * u >= r1) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)xv[u][e];
      a[e] = fmaxf(a[e], v);
      m[e] = fminf(m[e], v);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    gmax[rg][8 * ch + e] = a[e];
    gmin[rg][8 * ch + e] = m[e];
  }
  __syncthreads();
  for (int d = tid; d < D; d += kRowThreads) {
    float mx = gmax[0][d], mn = gmin[0][d];
#pragma unroll
    for (int g = 1; g < RG; ++g) {
      mx = fmaxf(mx, gmax[g][d]);
      mn = fminf(mn, gmin[g][d]);
    }
    xs[d] = mx;
    xs[D + d] = mn;
  }
  __syncthreads();
  project_row<DG>(xs, 2 * D, wk + (size_t)(bg % Hkv) * 2 * D * DG, part, j, rope_base,
                  kt + ((size_t)bg * nkb + j) * DG);
}

// Scores of one (sequence, query head): the token's Q~ (project_row), logits
// scale <Q~, K~_j> over the blocks j < nb, then the softmax; a
// fixed reduction order, so results are bit-reproducible.  Blocks j >= nb get 0
// (a whole row when nb = 0).
constexpr int kDecGateThreads = 256;
constexpr int kDecGatePer = 4096 / kDecGateThreads;  // nKB <= 4096

// Workgroup L runs on XCD L % 8 (workgroups are dealt round-robin).  This maps
// L to an item so that XCD x gets the contiguous items x q + min(x, r) ..
// (q = N / 8, r = N % 8), a bijection of [0, N): the query heads of one KV
// group, which read the same gate keys, then share an XCD and its L2.
__device__ __forceinline__ int xcd_contiguous_item(int L, int N) {
  const int q = N / 8, r = N % 8, x = L % 8, k = L / 8;
  return x * q + min(x, r) + k;
}

// v read from another lane of its 16-lane row by a DPP control (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

struct DecGateShared {
  float red[kDecGateThreads / 64];
  float xs[kDecGateThreads];  // the token, D <= 128 entries used
};

// The probabilities of a row with nb > 0 into x[u] (block j = tid + 256 u; 0 for
// j >= nb).  Called by the whole workgroup; lrow (LDS, >= nb floats) holds the
// logits on the way.  The logits are read with eight lanes per gate key, each
// lane taking every eighth 16-byte chunk of it, so one wave load covers eight
// whole rows; a lane sums its chunks in order and the eight partial sums are
// then added pairwise ((l0 + l1) + (l2 + l3)) + ((l4 + l5) + (l6 + l7)).
template <int DG>
__device__ __forceinline__ void decode_gate_probs(
    const __bf16* __restrict__ q, const float* __restrict__ wq, float rope_base, int D,
    const float* __restrict__ kt, int bh, int h, int kvrow, int nb, int nkb, float scale,
    float* qs, float (*part)[2][DG / 2], DecGateShared& sh, float* lrow,
    float (&x)[kDecGatePer]) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int V = DG / 32;    // 16-byte chunks per lane and key
  constexpr int U = 48 / V;     // keys per lane and batch: 48 loads in flight
  constexpr int kRowsPerPass = 8 * (kDecGateThreads / 64);
  const int sub = lane & 7;
  const int r0 = wv * 8 + (lane >> 3);
  const float* kr = kt + (size_t)kvrow * nkb * DG;  // uniform base, 32-bit lane offsets
  f32x4 kv[U][V];
  auto fetch = [&](int base) {  // rows past nb - 1 re-read row nb - 1 (unused)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = (uint32_t)min(base + kRowsPerPass * u + r0, nb - 1);
#pragma unroll
      for (int t = 0; t < V; ++t)
        kv[u][t] = *reinterpret_cast<const f32x4*>(kr + (j * DG + 32 * t + 4 * sub));
    }
  };
  // Q~ of the token (no pooling): q Wq[h], rotated at block nb - 1, into LDS.  The
  // token (D <= 128 < 256 threads) is requested first, then the first batch of gate
  // keys, which does not depend on Q~ and loads during the projection.
  const __bf16 qx = q[(size_t)bh * D + min(tid, D - 1)];  // in bounds, no branch
  fetch(0);
  sh.xs[tid] = (float)qx;  // entries D.. are not read
  __syncthreads();
  project_row<DG>(sh.xs, D, wq + (size_t)h * D * DG, part, nb - 1, rope_base, qs);
  f32x4 qv[V];
#pragma unroll
  for (int t = 0; t < V; ++t) qv[t] = *reinterpret_cast<const f32x4*>(qs + 4 * (sub + 8 * t));
  for (int base = 0; base < nb; base += kRowsPerPass * U) {
    if (base > 0) fetch(base);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < V; ++t) {
        s = fmaf(qv[t][0], kv[u][t][0], s);
        s = fmaf(qv[t][1], kv[u][t][1], s);
        s = fmaf(qv[t][2], kv[u][t][2], s);
        s = fmaf(qv[t][3], kv[u][t][3], s);
      }
      // Sum over the 8 lanes of the key: lane pairs, then quads (DPP quad
      // permutations), then the two quads (half-row mirror); every lane of the
      // group ends with the same bits.
      s += dpp_f32<0xB1>(s);   // quad_perm [1, 0, 3, 2]
      s += dpp_f32<0x4E>(s);   // quad_perm [2, 3, 0, 1]
      s += dpp_f32<0x141>(s);  // row_half_mirror
      const int j = base + kRowsPerPass * u + r0;
      if (sub == 0 && j < nb) lrow[j] = s * scale;
    }
  }
  __syncthreads();
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < kDecGatePer; ++u) {
    const int j = tid + kDecGateThreads * u;
    x[u] = -INFINITY;
    if (j < nb) {
      x[u] = lrow[j];
      mx = fmaxf(mx, x[u]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) sh.red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(sh.red[0], sh.red[1]), fmaxf(sh.red[2], sh.red[3]));
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int u = 0; u < kDecGatePer; ++u) {
    const int j = tid + kDecGateThreads * u;
    x[u] = j < nb ? expf(x[u] - mx) : 0.f;
    l += x[u];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
  if (lane == 0) sh.red[wv] = l;
  __syncthreads();
  l = ((sh.red[0] + sh.red[1]) + sh.red[2]) + sh.red[3];
  const float inv = 1.0f / l;
#pragma unroll
  for (int u = 0; u < kDecGatePer; ++u) x[u] *= inv;
}

template <int DG>
__global__ __launch_bounds__(kDecGateThreads) void gate_decode_scores_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ wq, float rope_base, int D,
    const float* __restrict__ kt, const int32_t* __restrict__ kv_len, int Hq, int Hkv, int Tmax,
    int bs, int nkb, float scale, float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) float qs[DG];
  __shared__ float part[kDecGateThreads / 64][2][DG / 2];
  __shared__ DecGateShared sh;
  __shared__ float lrow[4096];
  const int bh = xcd_contiguous_item(blockIdx.x, gridDim.x);  // b * Hq + h
  const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int len = min(max(kv_len[b], 0), Tmax);
  const int nb = len > 0 ? (len - 1) / bs + 1 : 0;
  float* out = scores + (size_t)bh * nkb;
  if (nb == 0) {
    for (int j = tid; j < nkb; j += kDecGateThreads) out[j] = 0.f;
    return;
  }
  float x[kDecGatePer];
  decode_gate_probs<DG>(q, wq, rope_base, D, kt, bh, h, b * Hkv + g, nb, nkb, scale, qs, part,
                        sh, lrow, x);
#pragma unroll
  for (int u = 0; u < kDecGatePer; ++u) {
    const int j = tid + kDecGateThreads * u;
    if (j < nkb) out[j] = x[u];  // 0 past the sequence
  }
}

// Scores and the decode block lists of one (sequence, query head) in one pass:
// the probabilities as gate_decode_scores_kernel computes them, optionally
// written out, then staged in LDS so that wave 0 holds block j = 64 c + lane in
// slot c and runs the selection of seer_build_mask_decode's decode rows (same
// keys, same count rule, same select): the same lists, bit for bit.
template <int DG, int NPL>
__global__ __launch_bounds__(kDecGateThreads) void gate_decode_mask_kernel(
    const __bf16* __restrict__ q, const float* __restrict__ wq, float rope_base, int D,
    const float* __restrict__ kt, const int32_t* __restrict__ kv_len, int Hq, int Hkv, int Tmax,
    int bs, int nkb, float scale, float* __restrict__ scores, int mode, float tau, int k_blocks,
    int keep_sink, int32_t* __restrict__ idx, int32_t* __restrict__ cnt, int max_k) {
  __shared__ __attribute__((aligned(16))) float qs[DG];
  __shared__ float part[kDecGateThreads / 64][2][DG / 2];
  __shared__ DecGateShared sh;
  __shared__ float prow[64 * NPL];
  __shared__ int hist[256];
  const int bh = xcd_contiguous_item(blockIdx.x, gridDim.x);  // b * Hq + h
  const int b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int len = min(max(kv_len[b], 0), Tmax);
  const int nb = len > 0 ? (len - 1) / bs + 1 : 0;
  if (nb > 0) {
    float x[kDecGatePer];
    decode_gate_probs<DG>(q, wq, rope_base, D, kt, bh, h, b * Hkv + g, nb, nkb, scale, qs, part,
                          sh, prow, x);
#pragma unroll
    for (int u = 0; u < kDecGatePer; ++u) {
      const int j = tid + kDecGateThreads * u;
      if (j < nkb) {
        prow[j] = x[u];
        if (scores) scores[(size_t)bh * nkb + j] = x[u];
      }
    }
  } else if (scores) {
    for (int j = tid; j < nkb; j += kDecGateThreads) scores[(size_t)bh * nkb + j] = 0.f;
  }
  __syncthreads();
  if (tid >= 64) return;
  // Decode row rule: the last block holds the token (forced, like the diagonal),
  // block 0 too with keep_sink; TopK keeps min(nb, max(forced, k_blocks)).
  const int i = nb - 1;
  const int n = nb;
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
        const float p = prow[j];
        kj = (mode == 1 || p >= tau) ? rowsel::order_key(p) : 0u;
      }
    }
    key[c] = kj;
    npos += kj != 0u;
  }
  npos = rowsel::wave_sum(npos);
  int k;
  if (mode == 1) {
    const int forced = (i == 0) ? 1 : (keep_sink ? 2 : 1);
    k = min(i + 1, max(forced, k_blocks));
  } else {
    k = min(npos, max_k);
  }
  const int count = rowsel::wave_select_row<NPL>(key, n, k, npos, lane, hist,
                                                 idx + (size_t)bh * max_k, max_k);
  if (lane == 0) cnt[bh] = count;
}

}  // namespace

// Workspace (fp32): Q~ [B,Hq,nQB,Dg], K~ [B,Hkv,nQB,Dg], per-row tile (max, sum)
// [B,Hq,nQB,tiles] x 2, pooled Q [B,Hq,nQB,D] and pooled K [B,Hkv,nQB,2D] (D <= 128).
size_t attn_gate_workspace_floats(int B, int Hq, int Hkv, int nqb, int dg) {
  const size_t ntiles = (nqb + kTile - 1) / kTile;
  return ((size_t)B * Hq + (size_t)B * Hkv) * nqb * dg + 2 * (size_t)B * Hq * nqb * ntiles +
         ((size_t)B * Hq + 2 * (size_t)B * Hkv) * nqb * 128;
}

namespace {

// Pooling and the linear layers + block RoPE (Q~ and K~ at the start of ws);
// *part_out points at the room for the per-row (max, sum) pairs of the logit
// tiles in the workspace.
hipError_t gate_front(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                      const float* wq, const float* wk, int dg, float rope_base, float* ws,
                      float2** part_out, hipStream_t stream) {
  const int nqb = (T + kTile - 1) / kTile;
  float* qt = ws;
  float* kt = ws + (size_t)B * Hq * nqb * dg;
  const size_t nt = (nqb + kTile - 1) / kTile;
  float* pq = kt + (size_t)B * Hkv * nqb * dg + 2 * (size_t)B * Hq * nqb * nt;
  float* pk = pq + (size_t)B * Hq * nqb * D;
  const long long units = (long long)B * (Hq + Hkv) * nqb;
  const dim3 pgrid((unsigned)((units + kPoolWaves - 1) / kPoolWaves));
  if (D == 128)
    hipLaunchKernelGGL(gate_pool_kernel<128>, pgrid, dim3(64 * kPoolWaves), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, B, Hq, Hkv, T, nqb, pq, pk);
  else
    hipLaunchKernelGGL(gate_pool_kernel<64>, pgrid, dim3(64 * kPoolWaves), 0, stream,
                       (const __bf16*)q, (const __bf16*)k, B, Hq, Hkv, T, nqb, pq, pk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t prow_tiles = (size_t)B * (Hq + Hkv) * ((nqb + kProjTileRows - 1) / kProjTileRows);
#define SEER_GATE_PROJECT(DG)                                                                  \
  hipLaunchKernelGGL(gate_project_kernel<DG>, dim3((unsigned)(prow_tiles * ProjCfg<DG>::NG)),   \
                     dim3(64 * kProjWaves), 0, stream, pq, pk, B, Hq, Hkv, D, nqb, wq, wk,       \
                     rope_base, qt, kt)
  if (dg == 128) SEER_GATE_PROJECT(128);
  else if (dg == 64) SEER_GATE_PROJECT(64);
  else SEER_GATE_PROJECT(32);
#undef SEER_GATE_PROJECT
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  *part_out = reinterpret_cast<float2*>(kt + (size_t)B * Hkv * nqb * dg);
  return hipSuccess;
}

// The logit tiles of tile rows it0 .. it1 - 1 (R logit rows per head in
// `logits`, see gate_logits_kernel) and their per-row (max, sum) pairs.
hipError_t gate_logits(int B, int Hq, int Hkv, int nqb, int dg, float scale, const float* ws,
                       int it0, int it1, int R, float* logits, float2* part,
                       hipStream_t stream) {
  const float* qt = ws;
  const float* kt = ws + (size_t)B * Hq * nqb * dg;
  const int npairs = it1 * (it1 + 1) / 2 - it0 * (it0 + 1) / 2;
  const dim3 lgrid((unsigned)((size_t)B * Hq * npairs));
#define SEER_GATE_LOGITS(DG)                                                                   \
  hipLaunchKernelGGL(gate_logits_kernel<DG>, lgrid, dim3(kScoreThreads), 0, stream, qt, kt,    \
                     Hq, Hkv, nqb, scale, it0, npairs, R, logits, part)
  if (dg == 128) SEER_GATE_LOGITS(128);
  else if (dg == 64) SEER_GATE_LOGITS(64);
  else SEER_GATE_LOGITS(32);
#undef SEER_GATE_LOGITS
  return hipGetLastError();
}

// The one-pass gate's front (nQB <= kRowsMaxBlocks), two kernels: K~
// [B,Hkv,nQB,Dg] at the start of ws, then the pooled Q [B,Hq,nQB,D], then Q~
// [B,Hq,nQB,Dg].
hipError_t gate_pool_keys(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                          const float* wk, int dg, float rope_base, int qsplit, float* ws,
                          hipStream_t stream) {
  const int nqb = (T + kTile - 1) / kTile;
  float* kt = ws;
  float* pq = ws + (size_t)B * Hkv * nqb * dg;
  const size_t ng = (nqb + kPPRows - 1) / kPPRows;
  const size_t nq8 = (nqb - qsplit + kPPWaves - 1) / kPPWaves;
  const dim3 grid((unsigned)((size_t)B * Hkv * ng + (size_t)B * Hq * nq8));
  const RopeFreqs freqs = rope_freqs(rope_base, dg);
#define SEER_GATE_PP(DD, DG)                                                                   \
  hipLaunchKernelGGL((gate_pool_project_kernel<DD, DG>), grid, dim3(64 * kPPWaves), 0, stream, \
                     (const __bf16*)q, (const __bf16*)k, B, Hkv, T, nqb, qsplit, wk, freqs, \
                     pq, kt)
  if (D == 128) {
    if (dg == 128) SEER_GATE_PP(128, 128);
    else if (dg == 64) SEER_GATE_PP(128, 64);
    else SEER_GATE_PP(128, 32);
  } else {
    if (dg == 128) SEER_GATE_PP(64, 128);
    else if (dg == 64) SEER_GATE_PP(64, 64);
    else SEER_GATE_PP(64, 32);
  }
#undef SEER_GATE_PP
  return hipGetLastError();
}

// First query block whose Q the pooling kernel pools (the heavier groups, at or
// past it, then start their logits at once while the others pool).
int gate_qsplit(int nqb) {
  const int G = (nqb + kRowGroup - 1) / kRowGroup;
  return kRowGroup * (G * kGateSplitNum / kGateSplitDen);
}

template <int D, int DG, int NPL, bool MASK>
hipError_t gate_rows_launch(const void* q, int T, int qsplit, const float* wq,
                            const RopeFreqs& freqs, int B, int Hq, int Hkv, int nqb, float scale,
                            const float* ws,
                            float* scores, int mode, float tau, double density, int keep_sink,
                            int32_t* idx, int32_t* cnt, int max_k, hipStream_t stream) {
  const float* kt = ws;
  const float* pq = ws + (size_t)B * Hkv * nqb * DG;
  const int G = (nqb + kRowGroup - 1) / kRowGroup;
  const size_t lds = gate_rows_lds_bytes(nqb, D, DG);
  auto kern = gate_rows_kernel<D, DG, NPL, MASK>;
  if (lds > 65536) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)((size_t)B * Hq * G)), dim3(64 * kRowsWaves), lds,
                     stream, (const __bf16*)q, T, pq, qsplit, wq, freqs, kt, B * Hq, Hq, Hkv,
                     nqb, scale,
                     scores, mode, tau, density, keep_sink, idx, cnt, max_k);
  return hipGetLastError();
}

template <bool MASK>
hipError_t gate_rows(const void* q, int T, int D, int qsplit, const float* wq, float rope_base,
                     int B, int Hq, int Hkv, int nqb, int dg, float scale, const float* ws,
                     float* scores,
                     int mode, float tau, double density, int keep_sink, int32_t* idx,
                     int32_t* cnt, int max_k, hipStream_t stream) {
  const RopeFreqs freqs = rope_freqs(rope_base, dg);
#define SEER_GATE_ROWS_CALL(DD, DG, NPL)                                                      \
  return gate_rows_launch<DD, DG, NPL, MASK>(q, T, qsplit, wq, freqs, B, Hq, Hkv, nqb, scale, ws, \
                                             scores, mode, tau, density, keep_sink, idx, cnt, \
                                             max_k, stream)
#define SEER_GATE_ROWS_NPL(DD, DG)                     \
  do {                                                 \
    if (nqb <= 64) SEER_GATE_ROWS_CALL(DD, DG, 1);     \
    if (nqb <= 64 * 4) SEER_GATE_ROWS_CALL(DD, DG, 4); \
    if (nqb <= 64 * 8) SEER_GATE_ROWS_CALL(DD, DG, 8); \
    if (nqb <= 64 * 16) SEER_GATE_ROWS_CALL(DD, DG, 16); \
    SEER_GATE_ROWS_CALL(DD, DG, 32);                   \
  } while (0)
  static_assert(kRowsMaxBlocks == 64 * 32, "NPL ladder covers kRowsMaxBlocks");
  if (nqb > kRowsMaxBlocks) return hipErrorInvalidValue;
  if (D == 128) {
    if (dg == 128) SEER_GATE_ROWS_NPL(128, 128);
    if (dg == 64) SEER_GATE_ROWS_NPL(128, 64);
    SEER_GATE_ROWS_NPL(128, 32);
  }
  if (dg == 128) SEER_GATE_ROWS_NPL(64, 128);
  if (dg == 64) SEER_GATE_ROWS_NPL(64, 64);
  SEER_GATE_ROWS_NPL(64, 32);
#undef SEER_GATE_ROWS_NPL
#undef SEER_GATE_ROWS_CALL
}

}  // namespace

hipError_t launch_attn_gate(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                            const float* wq, const float* wk, int dg, float scale,
                            float rope_base, float* scores, float* ws, hipStream_t stream) {
  const int nqb = (T + kTile - 1) / kTile;
  if ((size_t)B * Hq * nqb == 0) return hipSuccess;
  if (nqb <= kRowsMaxBlocks) {
    const int qsplit = gate_qsplit(nqb);
    hipError_t err = gate_pool_keys(q, k, B, Hq, Hkv, T, D, wk, dg, rope_base, qsplit, ws, stream);
    if (err != hipSuccess) return err;
    return gate_rows<false>(q, T, D, qsplit, wq, rope_base, B, Hq, Hkv, nqb, dg, scale, ws, scores, 0,
                            0.f, 0.0, 0, nullptr,
                            nullptr, 1, stream);
  }
  float2* part = nullptr;
  hipError_t err = gate_front(q, k, B, Hq, Hkv, T, D, wq, wk, dg, rope_base, ws, &part, stream);
  if (err != hipSuccess) return err;
  const int ntiles = (nqb + kTile - 1) / kTile;
  err = gate_logits(B, Hq, Hkv, nqb, dg, scale, ws, 0, ntiles, nqb, scores, part, stream);
  if (err != hipSuccess) return err;
  const int rows = B * Hq * nqb;  // < 2^31: the host layer checks B (Hq + Hkv) nQB
  hipLaunchKernelGGL(gate_softmax_kernel, dim3((unsigned)((rows + kRowWaves - 1) / kRowWaves)),
                     dim3(64 * kRowWaves), 0, stream, rows, nqb, scores, part);
  return hipGetLastError();
}

hipError_t launch_attn_gate_mask(const void* q, const void* k, int B, int Hq, int Hkv, int T,
                                 int D, const float* wq, const float* wk, int dg, float scale,
                                 float rope_base, int mode, float threshold, double density,
                                 int keep_sink, int32_t* idx, int32_t* cnt, int max_k,
                                 float* scores, float* ws, int pass_rows, hipStream_t stream) {
  const int nqb = (T + kTile - 1) / kTile;
  if ((size_t)B * Hq * nqb == 0) return hipSuccess;
  if (nqb <= kRowsMaxBlocks) {  // the logits stay on chip: no passes, no logits buffer
    const int qsplit = gate_qsplit(nqb);
    hipError_t err = gate_pool_keys(q, k, B, Hq, Hkv, T, D, wk, dg, rope_base, qsplit, ws, stream);
    if (err != hipSuccess) return err;
    return gate_rows<true>(q, T, D, qsplit, wq, rope_base, B, Hq, Hkv, nqb, dg, scale, ws, scores, mode,
                           threshold, density, keep_sink, idx, cnt, max_k, stream);
  }
  // Without a scores buffer the logits live past the gate's own workspace, at
  // the next 256-byte boundary (within the 256 bytes of slack the workspace
  // size adds), pass_rows rows per head at a time.
  const size_t off = (attn_gate_workspace_floats(B, Hq, Hkv, nqb, dg) + 63) & ~(size_t)63;
  const int R = scores ? nqb : pass_rows;  // logit rows per head per pass
  float* logits = scores ? scores : ws + off;
  float2* part = nullptr;
  hipError_t err = gate_front(q, k, B, Hq, Hkv, T, D, wq, wk, dg, rope_base, ws, &part, stream);
  if (err != hipSuccess) return err;
  const int ntiles = (nqb + kTile - 1) / kTile;
  const int tiles_per_pass = R >= nqb ? ntiles : R / kTile;
  const int ws_flag = scores ? 1 : 0;
  for (int it0 = 0; it0 < ntiles; it0 += tiles_per_pass) {
    const int it1 = min(it0 + tiles_per_pass, ntiles);
    err = gate_logits(B, Hq, Hkv, nqb, dg, scale, ws, it0, it1, R, logits, part, stream);
    if (err != hipSuccess) return err;
    const int row0 = kTile * it0;
    const int Rv = min(kTile * it1, nqb) - row0;  // rows of this pass, per head
    const int rows = B * Hq * Rv;
    const dim3 grid((unsigned)((rows + kRowWaves - 1) / kRowWaves));
#define SEER_GATE_MASK(NPL)                                                                    \
  hipLaunchKernelGGL(gate_softmax_mask_kernel<NPL>, grid, dim3(64 * kRowWaves), 0, stream, rows, \
                     nqb, row0, Rv, R, logits, ws_flag, part, mode, threshold, density,          \
                     keep_sink, idx, cnt, max_k)
    if (nqb <= 64) SEER_GATE_MASK(1);
    else if (nqb <= 64 * 4) SEER_GATE_MASK(4);
    else if (nqb <= 64 * 8) SEER_GATE_MASK(8);
    else if (nqb <= 64 * 16) SEER_GATE_MASK(16);
    else if (nqb <= 64 * 32) SEER_GATE_MASK(32);
    else if (nqb <= 64 * 64) SEER_GATE_MASK(64);
    else return hipErrorInvalidValue;  // the host layer rejects nQB > 4096 first
#undef SEER_GATE_MASK
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Decode gate keys workspace (fp32): the pooled cache K [B,Hkv,nKB,2D].
size_t attn_gate_decode_keys_workspace_floats(int B, int Hkv, int nkb, int D) {
  return (size_t)B * Hkv * nkb * 2 * D;
}

hipError_t launch_attn_gate_decode_keys(const void* k, const int32_t* kv_len, int B, int Hkv,
                                        int Tmax, int D, const float* wk, int dg,
                                        float rope_base, int block, int only_last,
                                        float* kt, float* ws, hipStream_t stream) {
  const int nkb = (Tmax + block - 1) / block;
  if (B == 0) return hipSuccess;
  if (only_last) {
#define SEER_GATE_KLAST(DD, DG)                                                                \
  hipLaunchKernelGGL((gate_decode_last_key_kernel<DD, DG>), dim3((unsigned)(B * Hkv)),         \
                     dim3(kRowThreads), 0, stream, (const __bf16*)k, kv_len, Hkv, Tmax, nkb,     \
                     block, wk, rope_base, kt)
    if (D == 128) {
      if (dg == 128) SEER_GATE_KLAST(128, 128);
      else if (dg == 64) SEER_GATE_KLAST(128, 64);
      else SEER_GATE_KLAST(128, 32);
    } else {
      if (dg == 128) SEER_GATE_KLAST(64, 128);
      else if (dg == 64) SEER_GATE_KLAST(64, 64);
      else SEER_GATE_KLAST(64, 32);
    }
#undef SEER_GATE_KLAST
    return hipGetLastError();
  }
  float* pk = ws;
  const int units = B * Hkv * nkb;  // < 2^31: checked by the host layer
  const dim3 pgrid((unsigned)((units + kPoolWaves - 1) / kPoolWaves));
  if (D == 128)
    hipLaunchKernelGGL(gate_decode_pool_kernel<128>, pgrid, dim3(64 * kPoolWaves), 0, stream,
                       (const __bf16*)k, kv_len, B, Hkv, Tmax, nkb, block, pk);
  else
    hipLaunchKernelGGL(gate_decode_pool_kernel<64>, pgrid, dim3(64 * kPoolWaves), 0, stream,
                       (const __bf16*)k, kv_len, B, Hkv, Tmax, nkb, block, pk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // Every block slot on the matrix cores (slots past a sequence hold stale pooled
  // rows; their K~ rows are never read).
  const size_t prow_tiles = (size_t)B * Hkv * ((nkb + kProjTileRows - 1) / kProjTileRows);
#define SEER_GATE_KPROJ(DG)                                                                    \
  hipLaunchKernelGGL(gate_project_kernel<DG>, dim3((unsigned)(prow_tiles * ProjCfg<DG>::NG)),   \
                     dim3(64 * kProjWaves), 0, stream, nullptr, pk, B, 0, Hkv, D, nkb, nullptr,  \
                     wk, rope_base, nullptr, kt)
  if (dg == 128) SEER_GATE_KPROJ(128);
  else if (dg == 64) SEER_GATE_KPROJ(64);
  else SEER_GATE_KPROJ(32);
#undef SEER_GATE_KPROJ
  return hipGetLastError();
}

hipError_t launch_attn_gate_decode_scores(const void* q, const float* kt, const int32_t* kv_len,
                                          int B, int Hq, int Hkv, int Tmax, int D,
                                          const float* wq, int dg, float scale, float rope_base,
                                          int block, float* scores, hipStream_t stream) {
  const int nkb = (Tmax + block - 1) / block;
  if (B == 0) return hipSuccess;
#define SEER_GATE_DSC(DG)                                                                      \
  hipLaunchKernelGGL(gate_decode_scores_kernel<DG>, dim3((unsigned)(B * Hq)),                   \
                     dim3(kDecGateThreads), 0, stream, (const __bf16*)q, wq, rope_base, D, kt,  \
                     kv_len, Hq, Hkv, Tmax, block, nkb, scale, scores)
  if (dg == 128) {
    SEER_GATE_DSC(128);
  } else if (dg == 64) {
    SEER_GATE_DSC(64);
  } else {
    SEER_GATE_DSC(32);
  }
#undef SEER_GATE_DSC
  return hipGetLastError();
}

hipError_t launch_attn_gate_decode_mask(const void* q, const float* kt, const int32_t* kv_len,
                                        int B, int Hq, int Hkv, int Tmax, int D, const float* wq,
                                        int dg, float scale, float rope_base, int block,
                                        int mode, float threshold, int k_blocks, int keep_sink,
                                        int32_t* idx, int32_t* cnt, int max_k, float* scores,
                                        hipStream_t stream) {
  const int nkb = (Tmax + block - 1) / block;
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)(B * Hq));
#define SEER_DGM(DG, NPL)                                                                      \
  hipLaunchKernelGGL((gate_decode_mask_kernel<DG, NPL>), grid, dim3(kDecGateThreads), 0, stream, \
                     (const __bf16*)q, wq, rope_base, D, kt, kv_len, Hq, Hkv, Tmax, block, nkb,  \
                     scale, scores, mode, threshold, k_blocks, keep_sink, idx, cnt, max_k)
#define SEER_DGM_NPL(DG)                                                                       \
  if (nkb <= 64) SEER_DGM(DG, 1);                                                              \
  else if (nkb <= 64 * 4) SEER_DGM(DG, 4);                                                     \
  else if (nkb <= 64 * 8) SEER_DGM(DG, 8);                                                     \
  else if (nkb <= 64 * 16) SEER_DGM(DG, 16);                                                   \
  else if (nkb <= 64 * 32) SEER_DGM(DG, 32);                                                   \
  else SEER_DGM(DG, 64)
  if (dg == 128) {
    SEER_DGM_NPL(128);
  } else if (dg == 64) {
    SEER_DGM_NPL(64);
  } else {
    SEER_DGM_NPL(32);
  }
#undef SEER_DGM_NPL
#undef SEER_DGM
  return hipGetLastError();
}

}  // namespace seer
