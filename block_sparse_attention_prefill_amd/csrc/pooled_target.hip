// Row-normalised distillation target and its MSE against gate scores.
//
// The max-pooled attention map is normalised per row so that, like the gate's
// softmax output, each row sums to 1 (rebuttal "SeerAttention: Learning
// Intrinsic Sparse Attention in Your LLMs", "Question 2: (Row-Normalization of
// Max-Pooled Attention Map)"), and the gate is trained against it with an MSE
// loss (same rebuttal, "Question 2 (Currently use MSE loss, how about e2e LM
// loss?)").  Rows hold the causal entries j <= i; entries above the diagonal
// are written as 0 and never read.
//
// HBM-bound: one wave64 per map row reads the row once to sum it and once more
// to normalise (the second read hits L2), with coalesced 16-byte lanes when
// the rows allow it (4-byte lanes otherwise).  The sums use a fixed reduction
// order, so results are bit-reproducible.
#include "seer_internal.h"

namespace seer {
namespace {

constexpr int kWaves = 4;
constexpr int kLossThreads = 1024;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Row value of the target: a / s for a causal entry of a row whose sum s is
// positive, else 0.
__device__ __forceinline__ float norm_entry(float a, float s) { return s > 0.f ? a / s : 0.f; }

// Scalar form: any nQB and any 4-byte alignment.
__global__ __launch_bounds__(64 * kWaves) void pooled_target_kernel(
    const float* amap, const float* __restrict__ gate, int rows, int nqb, float* target,
    float* __restrict__ row_sse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = row % nqb;
  const float* a = amap + row * (long long)nqb;
  float* t = target + row * (long long)nqb;
  float s = 0.f;
  for (int j = lane; j <= i; j += 64) s += a[j];
  s = wave_sum(s);  // every lane's reads of the row are done past this point
  float e = 0.f;
  for (int j = lane; j < nqb; j += 64) {
    float v = 0.f;
    if (j <= i) {
      v = norm_entry(a[j], s);
      if (gate) {
        const float d = gate[row * (long long)nqb + j] - v;
        e = fmaf(d, d, e);
      }
    }
    t[j] = v;
  }
  if (gate && row_sse) {
    e = wave_sum(e);
    if (lane == 0) row_sse[row] = e;
  }
}

// 16-byte form (nQB % 4 == 0, all rows 16-byte aligned): lane L takes the
// 4-float chunks L, L + 64, ...; chunks wholly inside j <= i move as one
// 16-byte access, the chunk the diagonal cuts is read element by element so
// that no entry j > i is read, and the chunks past it are written as zeros.
// In place is safe: every chunk is read and written by the same lane, reads
// first.
__global__ __launch_bounds__(64 * kWaves) void pooled_target_vec_kernel(
    const float* amap, const float* __restrict__ gate, int rows, int nqb, float* target,
    float* __restrict__ row_sse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = row % nqb;
  const int nch = nqb >> 2;
  const int full = (i + 1) >> 2;  // chunks 0 .. full - 1 lie wholly in j <= i
  const int rem = (i + 1) & 3;    // causal entries of chunk `full`
  const float* a = amap + row * (long long)nqb;
  const float4* a4 = reinterpret_cast<const float4*>(a);
  float s = 0.f;
  for (int c = lane; c < full; c += 64) {
    const float4 x = a4[c];
    s += (x.x + x.y) + (x.z + x.w);
  }
  if (rem && lane == (full & 63))
    for (int u = 0; u < rem; ++u) s += a[4 * full + u];
  s = wave_sum(s);  // every lane's reads of the row are done past this point
  float4* t4 = reinterpret_cast<float4*>(target + row * (long long)nqb);
  const float* g = gate ? gate + row * (long long)nqb : nullptr;
  float e = 0.f;
  for (int c = lane; c < nch; c += 64) {
    float4 v = {0.f, 0.f, 0.f, 0.f};
    if (c < full) {
      const float4 x = a4[c];
      v = {norm_entry(x.x, s), norm_entry(x.y, s), norm_entry(x.z, s), norm_entry(x.w, s)};
      if (g) {
        const float4 y = reinterpret_cast<const float4*>(g)[c];
        const float d0 = y.x - v.x, d1 = y.y - v.y, d2 = y.z - v.z, d3 = y.w - v.w;
        e = fmaf(d0, d0, e);
        e = fmaf(d1, d1, e);
        e = fmaf(d2, d2, e);
        e = fmaf(d3, d3, e);
      }
    } else if (c == full && rem) {
      float w[4] = {0.f, 0.f, 0.f, 0.f};
      for (int u = 0; u < rem; ++u) {
        w[u] = norm_entry(a[4 * c + u], s);
        if (g) {
          const float d = g[4 * c + u] - w[u];
          e = fmaf(d, d, e);
        }
      }
      v = {w[0], w[1], w[2], w[3]};
    }
    t4[c] = v;
  }
  if (gate && row_sse) {
    e = wave_sum(e);
    if (lane == 0) row_sse[row] = e;
  }
}

// 16-byte form with the row held in registers (nQB <= 256 NC): the causal
// chunks of the map and of the gate are all requested before the row sum, so a
// row costs one memory round trip; the map is read once.  Same chunk rules as
// above.
template <int NC>
__global__ __launch_bounds__(64 * kWaves) void pooled_target_reg_kernel(
    const float* amap, const float* __restrict__ gate, int rows, int nqb, float* target,
    float* __restrict__ row_sse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = row % nqb;
  const int nch = nqb >> 2;
  const int full = (i + 1) >> 2;
  const int rem = (i + 1) & 3;
  const float* a = amap + row * (long long)nqb;
  const float* g = gate ? gate + row * (long long)nqb : nullptr;
  const float4 zero = {0.f, 0.f, 0.f, 0.f};
  float4 x[NC], y[NC];
  // Every load is issued before any is used and none sits under a per-lane
  // branch (each would be waited for on its own): chunks past the last full
  // one re-read it, the partial chunk's entries are re-read from entries <= i,
  // and selects drop what is not the row's.  No entry j > i is read.
  const float4* a4 = reinterpret_cast<const float4*>(a);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const int clast = max(full - 1, 0);
  float4 xl[NC], yl[NC];
  if (full > 0) {
#pragma unroll
    for (int u = 0; u < NC; ++u) xl[u] = a4[min(lane + 64 * u, clast)];
    if (g) {
#pragma unroll
      for (int u = 0; u < NC; ++u) yl[u] = g4[min(lane + 64 * u, clast)];
    }
  }
  float xr[3], yr[3] = {0.f, 0.f, 0.f};  // entries 4 full + k of the partial chunk
#pragma unroll
  for (int k = 0; k < 3; ++k) xr[k] = a[min(4 * full + k, i)];
  if (g) {
#pragma unroll
    for (int k = 0; k < 3; ++k) yr[k] = g[min(4 * full + k, i)];
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = lane + 64 * u;
    x[u] = zero;
    y[u] = zero;
    if (c < full) {
      x[u] = xl[u];
      if (g) y[u] = yl[u];
    } else if (c == full && rem) {
      x[u] = {xr[0], rem > 1 ? xr[1] : 0.f, rem > 2 ? xr[2] : 0.f, 0.f};
      y[u] = {yr[0], rem > 1 ? yr[1] : 0.f, rem > 2 ? yr[2] : 0.f, 0.f};
    }
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < NC; ++u) s += (x[u].x + x[u].y) + (x[u].z + x[u].w);
  s = wave_sum(s);  // every lane's reads of the row are done past this point
  float4* t4 = reinterpret_cast<float4*>(target + row * (long long)nqb);
  float e = 0.f;
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = lane + 64 * u;
    if (c >= nch) break;
    // Entries past the diagonal hold 0 in x and y: their target is 0 and their
    // error term (0 - 0)^2 adds nothing.
    const float4 v = {norm_entry(x[u].x, s), norm_entry(x[u].y, s), norm_entry(x[u].z, s),
                      norm_entry(x[u].w, s)};
    if (g) {
      const float d0 = y[u].x - v.x, d1 = y[u].y - v.y, d2 = y[u].z - v.z, d3 = y[u].w - v.w;
      e = fmaf(d0, d0, e);
      e = fmaf(d1, d1, e);
      e = fmaf(d2, d2, e);
      e = fmaf(d3, d3, e);
    }
    t4[c] = v;
  }
  if (gate && row_sse) {
    e = wave_sum(e);
    if (lane == 0) row_sse[row] = e;
  }
}

// Mean of the per-row squared errors over all causal entries; one workgroup,
// fixed summation order.
__global__ __launch_bounds__(kLossThreads) void mse_loss_kernel(const float* __restrict__ row_sse,
                                                              long long rows, double count,
                                                              float* __restrict__ loss) {
  __shared__ double part[kLossThreads / 64];
  // 32 independent loads in flight per thread (indices past the end re-read
  // the last row and are dropped by a select, so no load is predicated); the
  // additions keep the fixed order r = tid, tid + 1024, ...
  constexpr int kBatch = 32;
  double s = 0.0;
  for (long long r0 = threadIdx.x; r0 < rows; r0 += (long long)kBatch * kLossThreads) {
    float x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const long long r = r0 + (long long)u * kLossThreads;
      x[u] = row_sse[r < rows ? r : rows - 1];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      s += r0 + (long long)u * kLossThreads < rows ? (double)x[u] : 0.0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kLossThreads / 64; ++w) t += part[w];
    loss[0] = (float)(t / count);
  }
}

}  // namespace

hipError_t launch_pooled_target(const float* amap, const float* gate, int B, int H, int nqb,
                                float* target, float* row_sse, float* loss, hipStream_t stream) {
  const long long rows = (long long)B * H * nqb;
  if (rows == 0) return hipSuccess;
  const bool vec = nqb % 4 == 0 &&
                   (((uintptr_t)amap | (uintptr_t)gate | (uintptr_t)target) & 15) == 0;
  auto kernel = pooled_target_kernel;
  if (vec) {
    const int per_lane = (nqb / 4 + 63) / 64;  // 16-byte chunks per lane
    kernel = per_lane <= 2   ? pooled_target_reg_kernel<2>
             : per_lane <= 4 ? pooled_target_reg_kernel<4>
             : per_lane <= 8 ? pooled_target_reg_kernel<8>
                             : pooled_target_vec_kernel;
  }
  // rows < 2^31: the host layer checks B H nQB.
  hipLaunchKernelGGL(kernel, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(64 * kWaves),
                     0, stream, amap, gate, (int)rows, nqb, target, row_sse);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !loss) return err;
  const double count = (double)B * H * ((double)nqb * (nqb + 1) / 2);
  hipLaunchKernelGGL(mse_loss_kernel, dim3(1), dim3(kLossThreads), 0, stream, row_sse, rows, count,
                     loss);
  return hipGetLastError();
}

}  // namespace seer
