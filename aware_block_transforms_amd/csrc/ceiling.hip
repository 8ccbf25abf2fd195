// Matrix-core ceilings of this part, measured rather than taken from the data
// sheet: streams of independent MFMAs with their operands held in registers,
// one wave per SIMD, no memory traffic inside the timed loop.  Built into its
// own library (libwush_ceiling.so), not into libwush: these kernels compute
// nothing of the method; they bound what the method's kernels can reach.
//
//  * FP4 block-scaled MFMA (16x16x128 and 32x32x64), the W4A4 matmul's
//    instruction, with operand bits taken from a caller buffer: random bytes
//    give the random-operand rate, zero bytes the zero-operand rate.  The gap
//    between the two is the chip's power limit, not a kernel property.
//  * fp32 MFMA 16x16x4, the dense transform's instruction, issued as NCHAIN
//    accumulation chains (2 chains of bs/4 steps is the transform's pattern),
//    optionally with NVALU independent vector FMAs issued between the MFMAs,
//    which shows how much vector-ALU work hides under the matrix core.
//
// Every kernel reduces its accumulators into `out` at the end so that nothing
// is dead code; `out` has one float per thread.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kAcc16 = 8;   // independent 16x16 accumulators per wave
constexpr int kAcc32 = 4;   // independent 32x32 accumulators per wave

template <bool BIG>
__global__ __launch_bounds__(256, 1) void fp4_stream(const uint32_t* __restrict__ bits, float* __restrict__ out,
                                                      int iters) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t* p = bits + (t & 1023) * 16;
  v8i a = {static_cast<int>(p[0]), static_cast<int>(p[1]), static_cast<int>(p[2]), static_cast<int>(p[3]), 0, 0, 0, 0};
  v8i b = {static_cast<int>(p[4]), static_cast<int>(p[5]), static_cast<int>(p[6]), static_cast<int>(p[7]), 0, 0, 0, 0};
  const int sa = static_cast<int>(p[8] & 0x7f7f7f7fu) | 0x40404040, sb = static_cast<int>(p[9] & 0x7f7f7f7fu) | 0x40404040;
  float sum = 0.0f;
  if constexpr (!BIG) {
    v4f acc[kAcc16];
#pragma unroll
    for (int i = 0; i < kAcc16; ++i) acc[i] = v4f{static_cast<float>(i), 0.f, 0.f, 0.f};   // distinct, never merged
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < kAcc16; ++i)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i], 4, 4, 0, sa, 0, sb);
    }
#pragma unroll
    for (int i = 0; i < kAcc16; ++i) sum += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  } else {
    v16f acc[kAcc32];
#pragma unroll
    for (int i = 0; i < kAcc32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] = e ? 0.0f : static_cast<float>(i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < kAcc32; ++i)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 4, 4, 0, sa, 0, sb);
    }
#pragma unroll
    for (int i = 0; i < kAcc32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[i][e];
  }
  out[t] = sum;
}

// NCHAIN chains of 8 dependent fp32 16x16x4 MFMAs per iteration (the dense
// transform's step pattern at bs 32), with NVALU independent vector FMAs
// placed between them.
template <int NCHAIN, int NVALU>
__global__ __launch_bounds__(256) void f32_stream(const float* __restrict__ src, float* __restrict__ out, int iters) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const float* p = src + (t & 1023) * 16;
  float a[8], b[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) { a[c] = p[c]; b[c] = p[8 + c]; }
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = p[k] * 0.5f;
  float sum = 0.0f;
  for (int it = 0; it < iters; ++it) {
    // operands look new to the compiler every iteration, so the chains are
    // neither hoisted out of the loop nor merged (they start from distinct values)
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(a[c]), "+v"(b[c]));
    v4f acc[NCHAIN > 0 ? NCHAIN : 1];
#pragma unroll
    for (int h = 0; h < (NCHAIN > 0 ? NCHAIN : 1); ++h) acc[h] = v4f{static_cast<float>(h), 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int h = 0; h < NCHAIN; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c], b[c], acc[h], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < NVALU; ++k) v[k & 7] = __builtin_fmaf(v[k & 7], 0.999f, 0.001f);
    }
#pragma unroll
    for (int h = 0; h < NCHAIN; ++h) sum += acc[h][0] + acc[h][3];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) sum += v[k];
  out[t] = sum;
}

template <typename K, typename... A>
int launch(K k, int blocks, void* stream, A... args) {
  hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), args...);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

// which: 0 = 16x16x128, 1 = 32x32x64.  bits: >= 1024 * 16 uint32 of operand
// bits; out: blocks * 256 floats.  Returns 0 on a successful launch.
int wush_ceiling_fp4(int which, int blocks, int iters, const uint32_t* bits, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !bits || !out) return 1;
  return which ? launch(fp4_stream<true>, blocks, stream, bits, out, iters)
               : launch(fp4_stream<false>, blocks, stream, bits, out, iters);
}

// fp32 16x16x4 with nchain in {2, 8} chains and nvalu in {0, 4, 8} vector FMAs per step.
int wush_ceiling_f32(int nchain, int nvalu, int blocks, int iters, const float* src, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !src || !out) return 1;
  if (nchain == 2 && nvalu == 0) return launch(f32_stream<2, 0>, blocks, stream, src, out, iters);
  if (nchain == 2 && nvalu == 4) return launch(f32_stream<2, 4>, blocks, stream, src, out, iters);
  if (nchain == 2 && nvalu == 8) return launch(f32_stream<2, 8>, blocks, stream, src, out, iters);
  if (nchain == 8 && nvalu == 0) return launch(f32_stream<8, 0>, blocks, stream, src, out, iters);
  if (nchain == 8 && nvalu == 8) return launch(f32_stream<8, 8>, blocks, stream, src, out, iters);
  if (nchain == 0 && nvalu == 8) return launch(f32_stream<0, 8>, blocks, stream, src, out, iters);
  return 1;
}

}  // extern "C"
