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
// to normalise (the second read hits L2), with coalesced 4-byte lanes.  The
// sums use a fixed reduction order, so results are bit-reproducible.
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

__global__ __launch_bounds__(64 * kWaves) void pooled_target_kernel(
    const float* __restrict__ amap, const float* __restrict__ gate, long long rows, int nqb,
    float* target, float* __restrict__ row_sse) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = (int)(row % nqb);
  const float* a = amap + row * (long long)nqb;
  float* t = target + row * (long long)nqb;
  float s = 0.f;
  for (int j = lane; j <= i; j += 64) s += a[j];
  s = wave_sum(s);  // every lane's reads of the row are done past this point
  float e = 0.f;
  for (int j = lane; j < nqb; j += 64) {
    float v = 0.f;
    if (j <= i) {
      v = s > 0.f ? a[j] / s : 0.f;
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

// Mean of the per-row squared errors over all causal entries; one workgroup,
// fixed summation order.
__global__ __launch_bounds__(kLossThreads) void mse_loss_kernel(const float* __restrict__ row_sse,
                                                              long long rows, double count,
                                                              float* __restrict__ loss) {
  __shared__ double part[kLossThreads / 64];
  double s = 0.0;
  for (long long r = threadIdx.x; r < rows; r += kLossThreads) s += (double)row_sse[r];
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
  hipLaunchKernelGGL(pooled_target_kernel, dim3((unsigned)((rows + kWaves - 1) / kWaves)),
                     dim3(64 * kWaves), 0, stream, amap, gate, rows, nqb, target, row_sse);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !loss) return err;
  const double count = (double)B * H * ((double)nqb * (nqb + 1) / 2);
  hipLaunchKernelGGL(mse_loss_kernel, dim3(1), dim3(kLossThreads), 0, stream, row_sse, rows, count,
                     loss);
  return hipGetLastError();
}

}  // namespace seer
