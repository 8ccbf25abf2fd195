// NVFP4 and INT4 W4A4 matmuls for gfx950 (the format sweep of the WUSH news
// article's experiments paragraph: MXFP4, NVFP4 and INT4 layer loss).
//
// Neither format has a native block-scaled matrix instruction on CDNA4 (the
// scaled FP4 MFMA takes one E8M0 scale per 32 values), so:
//  * NVFP4: every value e2m1 * e4m3 has at most 6 significant bits, so it is
//    dequantized exactly to bf16 in registers and fed to the bf16 MFMA
//    (16x16x32); the two fp32 tensor scales multiply the result once.
//  * INT4: each 32-group is one int8 MFMA (16x16x32) into a fresh int32,
//    which is exact; the group's fp16 scales multiply exactly in fp32
//    (11 + 11 significant bits) and the product is accumulated in fp32.
// Fragments are loaded straight from global memory into VGPRs; the weight
// fragment is the first MFMA operand so each lane ends with four consecutive
// output columns.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

constexpr int kWaveM = 64, kWaveN = 64, kTM = 4, kTN = 4;
constexpr int kBlockM = 128, kBlockN = 128;

// fp32 bit pattern of an E2M1 code (sign in bit 3).
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t c) {
  const uint32_t m = c & 7u;
  const uint32_t mag = (m & 6u) ? ((m + 252u) << 22) : ((m & 1u) ? 0x3f000000u : 0u);
  return mag | ((c & 8u) << 28);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  if (ex == 0) return static_cast<float>(m) * 0.001953125f;
  return __uint_as_float(((ex + 120u) << 23) | (m << 20));
}

// 8 E2M1 codes (one dword) times a block scale -> 8 exact bf16 values.
__device__ __forceinline__ v8bf decode8_nv(uint32_t w, float s) {
  v8s r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = __uint_as_float(e2m1_bits((w >> (4 * i)) & 15u)) * s;
    r[i] = static_cast<short>(__float_as_uint(v) >> 16);   // exact: <= 8 significant bits
  }
  return __builtin_bit_cast(v8bf, r);
}

__global__ __launch_bounds__(256) void gemm_nvfp4_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                         const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                         float gab, float* __restrict__ Y, int M, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m_base = blockIdx.y * kBlockM + (wave >> 1) * kWaveM;
  const int n_base = blockIdx.x * kBlockN + (wave & 1) * kWaveN;
  const int r16 = lane & 15, grp = lane >> 4;
  const size_t krow = static_cast<size_t>(K) / 2, srow = static_cast<size_t>(K) / 16;
  const uint8_t *ap[kTM], *sap[kTM], *bp[kTN], *sbp[kTN];
#pragma unroll
  for (int t = 0; t < kTM; ++t) {
    const int m = min(m_base + 16 * t + r16, M - 1);
    ap[t] = A + m * krow;
    sap[t] = SA + m * srow;
  }
#pragma unroll
  for (int t = 0; t < kTN; ++t) {
    const int n = min(n_base + 16 * t + r16, N - 1);
    bp[t] = B + n * krow;
    sbp[t] = SB + n * srow;
  }
  v4f acc[kTN][kTM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int kc = 0; kc < K / 128; ++kc) {
    // lane group g owns elements [32g, 32g + 32) of this 128-chunk = NVFP4 blocks 2g, 2g+1
    const size_t cb = static_cast<size_t>(kc) * 64 + grp * 16;
    const size_t so = static_cast<size_t>(kc) * 8 + grp * 2;
    uint4 xa[kTM], wb[kTN];
    float xs0[kTM], xs1[kTM], ws0[kTN], ws1[kTN];
#pragma unroll
    for (int t = 0; t < kTM; ++t) {
      xa[t] = *reinterpret_cast<const uint4*>(ap[t] + cb);
      xs0[t] = e4m3_value(sap[t][so]);
      xs1[t] = e4m3_value(sap[t][so + 1]);
    }
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      wb[t] = *reinterpret_cast<const uint4*>(bp[t] + cb);
      ws0[t] = e4m3_value(sbp[t][so]);
      ws1[t] = e4m3_value(sbp[t][so + 1]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v8bf xv[kTM], wv[kTN];
#pragma unroll
      for (int t = 0; t < kTM; ++t) {
        const uint32_t w = j == 0 ? xa[t].x : j == 1 ? xa[t].y : j == 2 ? xa[t].z : xa[t].w;
        xv[t] = decode8_nv(w, j < 2 ? xs0[t] : xs1[t]);
      }
#pragma unroll
      for (int t = 0; t < kTN; ++t) {
        const uint32_t w = j == 0 ? wb[t].x : j == 1 ? wb[t].y : j == 2 ? wb[t].z : wb[t].w;
        wv[t] = decode8_nv(w, j < 2 ? ws0[t] : ws1[t]);
      }
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int q = 0; q < kTM; ++q)
          acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[i], xv[q], acc[i][q], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < kTM; ++j) {
    const int m = m_base + 16 * j + r16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int n = n_base + 16 * i + 4 * grp;
      float* dst = Y + static_cast<size_t>(m) * N + n;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n + q < N) dst[q] = acc[i][j][q] * gab;
    }
  }
}

// 8 int4 codes (one dword) -> 8 sign-extended int8 in a 64-bit operand.
__device__ __forceinline__ long widen8_i4(uint32_t w) {
  uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
  lo |= (lo & 0x08080808u) * 30u;   // bytes >= 8 become b - 16 (0xf0 | b)
  hi |= (hi & 0x08080808u) * 30u;
  return static_cast<long>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ float f16_value(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

__global__ __launch_bounds__(256) void gemm_int4_kernel(const uint8_t* __restrict__ A, const uint16_t* __restrict__ SA,
                                                        const uint8_t* __restrict__ B, const uint16_t* __restrict__ SB,
                                                        float* __restrict__ Y, int M, int N, int K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m_base = blockIdx.y * kBlockM + (wave >> 1) * kWaveM;
  const int n_base = blockIdx.x * kBlockN + (wave & 1) * kWaveN;
  const int r16 = lane & 15, grp = lane >> 4;
  const size_t krow = static_cast<size_t>(K) / 2, srow = static_cast<size_t>(K) / 32;
  const uint8_t *ap[kTM], *bp[kTN];
  const uint16_t* sap[kTM];
  const uint16_t* sbo[kTN][4];   // weight scales of the 4 output columns this lane owns per tile
#pragma unroll
  for (int t = 0; t < kTM; ++t) {
    const int m = min(m_base + 16 * t + r16, M - 1);
    ap[t] = A + m * krow;
    sap[t] = SA + m * srow;
  }
#pragma unroll
  for (int t = 0; t < kTN; ++t) {
    const int n = min(n_base + 16 * t + r16, N - 1);
    bp[t] = B + n * krow;
#pragma unroll
    for (int q = 0; q < 4; ++q) sbo[t][q] = SB + min(n_base + 16 * t + 4 * grp + q, N - 1) * srow;
  }
  v4f acc[kTN][kTM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int g32 = 0; g32 < K / 32; ++g32) {
    // this MFMA covers exactly one 32-group; lane group g supplies its elements [8g, 8g + 8)
    const size_t cb = static_cast<size_t>(g32) * 16 + grp * 4;
    long xa[kTM], wb[kTN];
    float sa[kTM], sw[kTN][4];
#pragma unroll
    for (int t = 0; t < kTM; ++t) {
      xa[t] = widen8_i4(*reinterpret_cast<const uint32_t*>(ap[t] + cb));
      sa[t] = f16_value(sap[t][g32]);
    }
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      wb[t] = widen8_i4(*reinterpret_cast<const uint32_t*>(bp[t] + cb));
#pragma unroll
      for (int q = 0; q < 4; ++q) sw[t][q] = f16_value(sbo[t][q][g32]);
    }
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        const v4i r = __builtin_amdgcn_mfma_i32_16x16x32_i8(wb[i], xa[j], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] += static_cast<float>(r[q]) * (sa[j] * sw[i][q]);
      }
  }
#pragma unroll
  for (int j = 0; j < kTM; ++j) {
    const int m = m_base + 16 * j + r16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int n = n_base + 16 * i + 4 * grp;
      float* dst = Y + static_cast<size_t>(m) * N + n;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n + q < N) dst[q] = acc[i][j][q];
    }
  }
}

}  // namespace

namespace wush {

// Direct-load kernel: operands of 2^31 bytes or more (beyond the LDS kernel's
// 32-bit buffer offsets).
wush_status gemm_nvfp4_direct(int M, int N, int K, const uint8_t* A, const uint8_t* SA, float ga, const uint8_t* B,
                              const uint8_t* SB, float gb, float* Y, hipStream_t stream) {
  dim3 grid((N + kBlockN - 1) / kBlockN, (M + kBlockM - 1) / kBlockM);
  if (grid.y > 65535u) return fail(WUSH_E_SHAPE, "wush_w4a4_gemm: M too large");
  hipLaunchKernelGGL(gemm_nvfp4_kernel, grid, dim3(256), 0, stream, A, SA, B, SB, ga * gb, Y, M, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm (nvfp4) launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

// Direct-load kernel: operands of 2^31 bytes or more (beyond the LDS kernel's
// 32-bit buffer offsets).
wush_status gemm_int4_direct(int M, int N, int K, const uint8_t* A, const uint16_t* SA, const uint8_t* B,
                             const uint16_t* SB, float* Y, hipStream_t stream) {
  dim3 grid((N + kBlockN - 1) / kBlockN, (M + kBlockM - 1) / kBlockM);
  if (grid.y > 65535u) return fail(WUSH_E_SHAPE, "wush_w4a4_gemm: M too large");
  hipLaunchKernelGGL(gemm_int4_kernel, grid, dim3(256), 0, stream, A, SA, B, SB, Y, M, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm (int4) launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // namespace wush
