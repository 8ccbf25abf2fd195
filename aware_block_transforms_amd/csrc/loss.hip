// Layer loss of "WUSH: Near-Optimal Adaptive Transforms for LLM
// Quantization" (AI Radio), "Problem Setup and Goal": the squared L2 distance
// between the quantized layer output and the exact one, divided by
// d_out * batch.  Accumulated in fp64 in a fixed order (a fixed grid of
// partial sums, then one block summing the partials), so the result does not
// depend on scheduling.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

constexpr int kParts = 1024;
constexpr int kThreads = 256;

__device__ __forceinline__ double block_sum(double v, double* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) sh[t] += sh[t + s];
    __syncthreads();
  }
  return sh[0];
}

__global__ __launch_bounds__(kThreads) void loss_partial(const float* __restrict__ Yh, const float* __restrict__ Yr,
                                                         size_t total, double* __restrict__ part) {
  __shared__ double sh[kThreads];
  double acc = 0.0;
  const size_t stride = static_cast<size_t>(kParts) * kThreads;
  const size_t n4 = total / 4;
  const float4* h4 = reinterpret_cast<const float4*>(Yh);
  const float4* r4 = reinterpret_cast<const float4*>(Yr);
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += stride) {
    const float4 a = h4[i], b = r4[i];
    const double d0 = static_cast<double>(a.x) - b.x, d1 = static_cast<double>(a.y) - b.y;
    const double d2 = static_cast<double>(a.z) - b.z, d3 = static_cast<double>(a.w) - b.w;
    acc += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
  }
  for (size_t i = n4 * 4 + static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < total; i += stride) {
    const double d = static_cast<double>(Yh[i]) - Yr[i];
    acc += d * d;
  }
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void loss_final(const double* __restrict__ part, double count,
                                                       double* __restrict__ out) {
  __shared__ double sh[kThreads];
  double acc = 0.0;
  for (int i = threadIdx.x; i < kParts; i += kThreads) acc += part[i];
  const double s = block_sum(acc, sh);
  if (threadIdx.x == 0) *out = s / count;
}

}  // namespace

extern "C" {

size_t wush_loss_ws_bytes(int M, int N) {
  (void)M;
  (void)N;
  return sizeof(double) * kParts;
}

wush_status wush_layer_loss(int M, int N, const float* Yhat, const float* Yref, double* loss, void* ws,
                            void* stream) {
  if (!Yhat || !Yref || !loss || !ws) return wush::fail(WUSH_E_ARG, "wush_layer_loss: null pointer");
  if (M < 1 || N < 1) return wush::fail(WUSH_E_SHAPE, "wush_layer_loss: M and N must be >= 1");
  if (!wush::aligned16(Yhat) || !wush::aligned16(Yref) || (reinterpret_cast<uintptr_t>(ws) & 7u) ||
      (reinterpret_cast<uintptr_t>(loss) & 7u))
    return wush::fail(WUSH_E_ARG, "wush_layer_loss: misaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t total = static_cast<size_t>(M) * N;
  double* part = static_cast<double*>(ws);
  hipLaunchKernelGGL(loss_partial, dim3(kParts), dim3(kThreads), 0, s, Yhat, Yref, total, part);
  hipLaunchKernelGGL(loss_final, dim3(1), dim3(kThreads), 0, s, part, static_cast<double>(total), loss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_layer_loss launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // extern "C"
