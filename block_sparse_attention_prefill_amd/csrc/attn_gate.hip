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
// Four kernels:
// * gate_pool_kernel: one wave per (batch, head, 64-token block) pools the block
//   (16-byte loads all in flight, lane shuffles to combine).
// * gate_project_kernel: one workgroup per (batch, head, 16 blocks) applies the
//   head's linear layer (an LDS-tiled fp32 GEMM) and the block RoPE, whose
//   angles are formed in fp64 so that far block positions keep their accuracy.
// * gate_logits_kernel: one workgroup per causal 64 x 64 tile of block pairs
//   (LDS-tiled fp32 Q~ K~^T) writes the scaled logits and each row's tile max
//   and sum of exponentials; gate_softmax_kernel then combines a row's tile
//   pairs in a fixed order and normalises the row in place, zeros above the
//   diagonal.
#include "seer_internal.h"

#include <math.h>

namespace seer {
namespace {

constexpr int kProjThreads = 256;
constexpr int kScoreThreads = 256;
constexpr int kTile = 64;  // query and key blocks per scores tile; tokens per block
constexpr int kWRows = 32; // weight rows per LDS chunk of the linear layer
constexpr int kProjRows = 16;  // pooled rows (blocks) per projection workgroup

// Pooling: one wave per (batch, head slot, 64-token block).  Lane L reads
// 16-byte chunk L % C of rows L / C, L / C + 64 / C, ... (C = D / 8 chunks per
// row), all its loads in flight at once; lanes holding the same chunk are
// combined with shuffles.  Q heads are averaged into pq [B, Hq, nQB, D], KV
// heads max- and min-pooled into pk [B, Hkv, nQB, 2D] ([max | min]).
constexpr int kPoolWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kPoolWaves) void gate_pool_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, int B, int Hq, int Hkv, int T,
    int nqb, float* __restrict__ pq, float* __restrict__ pk) {
  constexpr int C = D / 8;          // chunks per row
  constexpr int R = 64 / C;         // rows read together by the wave
  constexpr int kPerLane = kTile / R;
  const int lane = threadIdx.x & 63;
  const long long unit = (long long)blockIdx.x * kPoolWaves + (threadIdx.x >> 6);
  if (unit >= (long long)B * (Hq + Hkv) * nqb) return;
  const int i = (int)(unit % nqb);
  const int bh = (int)(unit / nqb);  // b * (Hq + Hkv) + head slot
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
    if (r < r1) x[u] = *reinterpret_cast<const bf16x8*>(src + (size_t)r * D + 8 * ch);
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

// Linear layer + block RoPE: one workgroup per (batch, head slot, 16-block
// tile) computes the 16 x DG tile of pooled rows times the head's weights,
// streaming 32-row chunks of both through LDS (16-byte loads, issued before the
// barrier that frees the previous chunk).  Thread (ty, tx) owns row ty and
// columns tx + 16 c, which include both columns e and e + DG/2 of every RoPE
// pair it owns, so the rotation needs no exchange.  Angles are formed in fp64
// so that far block positions keep their accuracy.
template <int DG>
__global__ __launch_bounds__(kProjThreads) void gate_project_kernel(
    const float* __restrict__ pq, const float* __restrict__ pk, int B, int Hq, int Hkv, int D,
    int nqb, const float* __restrict__ wq, const float* __restrict__ wk, float rope_base,
    float* __restrict__ qt, float* __restrict__ kt) {
  constexpr int NC = DG / 16;  // columns per thread
  __shared__ __attribute__((aligned(16))) float as[kProjRows][kWRows];
  __shared__ __attribute__((aligned(16))) float ws[kWRows * DG];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // row ty, columns tx + 16 c
  const int ntiles = (nqb + kProjRows - 1) / kProjRows;
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int b = bh / (Hq + Hkv);
  const int slot = bh % (Hq + Hkv);
  const bool is_q = slot < Hq;
  const int head = is_q ? slot : slot - Hq;
  const int nheads = is_q ? Hq : Hkv;
  const int din = is_q ? D : 2 * D;
  const float* a = (is_q ? pq : pk) + ((size_t)b * nheads + head) * nqb * din;
  const float* w = (is_q ? wq : wk) + (size_t)head * din * DG;
  const int i0 = kProjRows * tile;
  constexpr int kWVec = kWRows * DG / 4 / kProjThreads;  // 16-byte weight loads per thread
  float acc[NC] = {};
  for (int d0 = 0; d0 < din; d0 += kWRows) {
    f32x4 va = {}, vw[kWVec];
    const int ar = tid / (kWRows / 4), ad = 4 * (tid % (kWRows / 4));  // 16 rows x 8 vectors
    if (tid < kProjRows * kWRows / 4 && i0 + ar < nqb)
      va = *reinterpret_cast<const f32x4*>(a + (size_t)(i0 + ar) * din + d0 + ad);
#pragma unroll
    for (int n = 0; n < kWVec; ++n)
      vw[n] = reinterpret_cast<const f32x4*>(w + (size_t)d0 * DG)[tid + kProjThreads * n];
    __syncthreads();  // the previous chunk has been used
    if (tid < kProjRows * kWRows / 4) *reinterpret_cast<f32x4*>(&as[ar][ad]) = va;
#pragma unroll
    for (int n = 0; n < kWVec; ++n) reinterpret_cast<f32x4*>(ws)[tid + kProjThreads * n] = vw[n];
    __syncthreads();
#pragma unroll 8
    for (int d = 0; d < kWRows; ++d) {
      const float av = as[ty][d];
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = fmaf(av, ws[d * DG + tx + 16 * c], acc[c]);
    }
  }
  const int i = i0 + ty;
  if (i >= nqb) return;
  float* out = (is_q ? qt : kt) + (((size_t)b * nheads + head) * nqb + i) * DG;
#pragma unroll
  for (int c = 0; c < NC / 2; ++c) {
    const int e = tx + 16 * c;  // e < DG / 2; its partner e + DG / 2 is column c + NC / 2
    const double ang = (double)i * pow((double)rope_base, -2.0 * e / (double)DG);
    const double cs = cos(ang), sn = sin(ang);
    const double x1 = acc[c], x2 = acc[c + NC / 2];
    out[e] = (float)(x1 * cs - x2 * sn);
    out[e + DG / 2] = (float)(x2 * cs + x1 * sn);
  }
}

// Logits of one 64 x 64 tile of (query block, key block) pairs, tile (it, jt)
// with jt <= it, enumerated per head in row-major lower-triangular order.
// Thread (ty, tx) of the 16 x 16 grid owns rows ty + 16 a and columns tx + 16 c
// (a, c = 0..3); the 16 threads of a row are 16 consecutive lanes, so row
// reductions are lane shuffles.  Writes the scaled logits (-inf above the
// diagonal) and, per row, the tile's max and sum of exp(logit - max).
template <int DG>
__global__ __launch_bounds__(kScoreThreads) void gate_logits_kernel(
    const float* __restrict__ qt, const float* __restrict__ kt, int Hq, int Hkv, int nqb,
    float scale, float* __restrict__ scores, float2* __restrict__ part) {
  __shared__ float qs[kTile][DG + 1];
  __shared__ float ks[kTile][DG + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int ntiles = (nqb + kTile - 1) / kTile;
  const int npairs = ntiles * (ntiles + 1) / 2;
  const int pair = blockIdx.x % npairs;
  const int bh = blockIdx.x / npairs;  // b * Hq + h
  int it = 0;
  while ((it + 1) * (it + 2) / 2 <= pair) ++it;
  const int jt = pair - it * (it + 1) / 2;
  const int b = bh / Hq;
  const int g = (bh % Hq) / (Hq / Hkv);
  const float* qrow = qt + (size_t)bh * nqb * DG;
  const float* krow = kt + ((size_t)b * Hkv + g) * nqb * DG;
  const int i0 = kTile * it, j0 = kTile * jt;
  {
    // Both 64 x DG tiles: 16-byte loads, all issued before the LDS stores.
    constexpr int kVec = kTile * DG / 4 / kScoreThreads;
    f32x4 vq[kVec], vk[kVec];
#pragma unroll
    for (int n = 0; n < kVec; ++n) {
      const int x = tid + kScoreThreads * n;
      const int r = x / (DG / 4), d4 = x % (DG / 4);
      vq[n] = (i0 + r < nqb) ? reinterpret_cast<const f32x4*>(qrow + (size_t)(i0 + r) * DG)[d4]
                             : f32x4{};
      vk[n] = (j0 + r < nqb) ? reinterpret_cast<const f32x4*>(krow + (size_t)(j0 + r) * DG)[d4]
                             : f32x4{};
    }
#pragma unroll
    for (int n = 0; n < kVec; ++n) {
      const int x = tid + kScoreThreads * n;
      const int r = x / (DG / 4), d = 4 * (x % (DG / 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qs[r][d + e] = vq[n][e];
        ks[r][d + e] = vk[n][e];
      }
    }
  }
  __syncthreads();
  float acc[4][4] = {};
#pragma unroll 4
  for (int d = 0; d < DG; ++d) {
    float qa[4], kc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) qa[a] = qs[ty + 16 * a][d];
#pragma unroll
    for (int c = 0; c < 4; ++c) kc[c] = ks[tx + 16 * c][d];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[a][c] = fmaf(qa[a], kc[c], acc[a][c]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty + 16 * a;
    float s[4];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tx + 16 * c;
      s[c] = (i < nqb && j <= i) ? acc[a][c] * scale : -INFINITY;
      mx = fmaxf(mx, s[c]);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tx + 16 * c;
      if (mx != -INFINITY && s[c] != -INFINITY) l += expf(s[c] - mx);
      if (i < nqb && j < nqb) scores[((size_t)bh * nqb + i) * nqb + j] = s[c];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) l += __shfl_xor(l, off, 64);
    if (tx == 0 && i < nqb) part[((size_t)bh * nqb + i) * ntiles + jt] = make_float2(mx, l);
  }
}

// One wave per score row: combine the row's per-tile (max, sum) pairs, then
// turn its logits into probabilities in place and zero the entries above the
// diagonal (including the tiles past the diagonal tile, never written above).
constexpr int kRowWaves = 4;

__global__ __launch_bounds__(64 * kRowWaves) void gate_softmax_kernel(
    long long rows, int nqb, float* __restrict__ scores, const float2* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = (int)(row % nqb);
  const int ntiles = (nqb + kTile - 1) / kTile;
  const int it = i / kTile;
  const float2* pr = part + row * ntiles;
  float m = -INFINITY, l = 0.f;
  for (int jt = 0; jt <= it; ++jt) {  // same order in every lane
    const float2 p = pr[jt];
    if (p.x == -INFINITY) continue;
    const float mn = fmaxf(m, p.x);
    l = (m == -INFINITY ? 0.f : l * expf(m - mn)) + p.y * expf(p.x - mn);
    m = mn;
  }
  const float inv = 1.0f / l;
  float* sr = scores + row * (long long)nqb;
  for (int j = lane; j < nqb; j += 64) sr[j] = (j <= i) ? expf(sr[j] - m) * inv : 0.f;
}

}  // namespace

// Workspace (fp32): Q~ [B,Hq,nQB,Dg], K~ [B,Hkv,nQB,Dg], per-row tile (max, sum)
// [B,Hq,nQB,tiles] x 2, pooled Q [B,Hq,nQB,D] and pooled K [B,Hkv,nQB,2D] (D <= 128).
size_t attn_gate_workspace_floats(int B, int Hq, int Hkv, int nqb, int dg) {
  const size_t ntiles = (nqb + kTile - 1) / kTile;
  return ((size_t)B * Hq + (size_t)B * Hkv) * nqb * dg + 2 * (size_t)B * Hq * nqb * ntiles +
         ((size_t)B * Hq + 2 * (size_t)B * Hkv) * nqb * 128;
}

hipError_t launch_attn_gate(const void* q, const void* k, int B, int Hq, int Hkv, int T, int D,
                            const float* wq, const float* wk, int dg, float scale,
                            float rope_base, float* scores, float* ws, hipStream_t stream) {
  const int nqb = (T + kTile - 1) / kTile;
  if ((size_t)B * Hq * nqb == 0) return hipSuccess;
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
  const dim3 jgrid((unsigned)((size_t)B * (Hq + Hkv) * ((nqb + kProjRows - 1) / kProjRows)));
#define SEER_GATE_PROJECT(DG)                                                                  \
  hipLaunchKernelGGL(gate_project_kernel<DG>, jgrid, dim3(kProjThreads), 0, stream, pq, pk, B, \
                     Hq, Hkv, D, nqb, wq, wk, rope_base, qt, kt)
  if (dg == 128) SEER_GATE_PROJECT(128);
  else if (dg == 64) SEER_GATE_PROJECT(64);
  else SEER_GATE_PROJECT(32);
#undef SEER_GATE_PROJECT
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ntiles = (nqb + kTile - 1) / kTile;
  const int npairs = ntiles * (ntiles + 1) / 2;
  float2* part = reinterpret_cast<float2*>(kt + (size_t)B * Hkv * nqb * dg);
  const dim3 lgrid((unsigned)((size_t)B * Hq * npairs));
#define SEER_GATE_LOGITS(DG)                                                                   \
  hipLaunchKernelGGL(gate_logits_kernel<DG>, lgrid, dim3(kScoreThreads), 0, stream, qt, kt,    \
                     Hq, Hkv, nqb, scale, scores, part)
  if (dg == 128) SEER_GATE_LOGITS(128);
  else if (dg == 64) SEER_GATE_LOGITS(64);
  else SEER_GATE_LOGITS(32);
#undef SEER_GATE_LOGITS
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long rows = (long long)B * Hq * nqb;
  hipLaunchKernelGGL(gate_softmax_kernel, dim3((unsigned)((rows + kRowWaves - 1) / kRowWaves)),
                     dim3(64 * kRowWaves), 0, stream, rows, nqb, scores, part);
  return hipGetLastError();
}

}  // namespace seer
