// MXFP4 x MXFP4 -> fp32 matmul on the gfx950 block-scaled FP4 matrix cores.
//
// "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization" (AI Radio),
// closing discussion: the per-layer speedup over BF16 comes from the FP4
// matmul of the transformed, quantized operands (W4A4).  WUSH news article,
// paragraph on experiments: MXFP4 = 32 E2M1 values sharing one E8M0 scale.
//
//   Y[m][n] = sum_b 2^(sa[m][b]-127) * 2^(sb[n][b]-127) * sum_{k in b} a[m][k] * w[n][k]
//
// Instruction: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in FP4
// (E2M1) and one E8M0 scale per lane (row or column, 32-element K group).
// For a 16x16x128 step lane l supplies row (l % 16) of its operand and the
// 32-element K group (l / 16), plus that group's scale byte.
//
// Operand roles: the weight fragment is the instruction's first operand and
// the activation fragment the second, so the 16x16 result holds Y^T: lane l
// ends up with Y[m0 + l%16][n0 + 4*(l/16) + 0..3], four consecutive output
// columns written with one 16-byte store.
//
// K ordering: a dot product may visit its K groups in any order as long as
// both operands agree, so the two MFMA sub-steps of a 256-wide K step give
// lane group g the K groups 2g and 2g+1: each lane then reads 32 contiguous
// code bytes and two contiguous scale bytes per row, and the scale byte for
// sub-step j is picked with op_sel.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaveM = 64;        // rows of Y per wave
constexpr int kWaveN = 64;        // cols of Y per wave
constexpr int kTM = kWaveM / 16;  // 16x16 tiles per wave along M
constexpr int kTN = kWaveN / 16;
constexpr int kBlockM = 2 * kWaveM;
constexpr int kBlockN = 2 * kWaveN;

__device__ __forceinline__ v8i as_operand(uint4 q) {
  v8i v = {static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w), 0, 0, 0, 0};
  return v;
}

template <int SEL>
__device__ __forceinline__ v4f mfma_fp4(uint4 w, uint32_t ws, uint4 x, uint32_t xs, v4f acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_operand(w), as_operand(x), acc, 4, 4, SEL,
                                                          static_cast<int>(ws), SEL, static_cast<int>(xs));
}

__global__ __launch_bounds__(256) void gemm_mxfp4_direct(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                         const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                         float* __restrict__ Y, int M, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m_base = blockIdx.y * kBlockM + (wave >> 1) * kWaveM;
  const int n_base = blockIdx.x * kBlockN + (wave & 1) * kWaveN;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  const size_t krow = static_cast<size_t>(K) / 2;    // code bytes per row
  const size_t srow = static_cast<size_t>(K) / 32;   // scale bytes per row

  const uint8_t* a_ptr[kTM];
  const uint8_t* sa_ptr[kTM];
  const uint8_t* b_ptr[kTN];
  const uint8_t* sb_ptr[kTN];
#pragma unroll
  for (int t = 0; t < kTM; ++t) {
    const int m = min(m_base + 16 * t + r16, M - 1);
    a_ptr[t] = A + m * krow;
    sa_ptr[t] = SA + m * srow;
  }
#pragma unroll
  for (int t = 0; t < kTN; ++t) {
    const int n = min(n_base + 16 * t + r16, N - 1);
    b_ptr[t] = B + n * krow;
    sb_ptr[t] = SB + n * srow;
  }

  v4f acc[kTN][kTM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int k256 = K / 256;
#pragma unroll 1
  for (int ks = 0; ks < k256; ++ks) {
    const size_t cb = static_cast<size_t>(ks) * 128 + grp * 32;   // code byte offset of this lane
    const size_t sbo = static_cast<size_t>(ks) * 8 + grp * 2;     // scale byte offset
    uint4 xa[kTM][2], wb[kTN][2];
    uint32_t xs[kTM], wsc[kTN];
#pragma unroll
    for (int t = 0; t < kTM; ++t) {
      const uint4* p = reinterpret_cast<const uint4*>(a_ptr[t] + cb);
      xa[t][0] = p[0];
      xa[t][1] = p[1];
      xs[t] = *reinterpret_cast<const uint16_t*>(sa_ptr[t] + sbo);
    }
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      const uint4* p = reinterpret_cast<const uint4*>(b_ptr[t] + cb);
      wb[t][0] = p[0];
      wb[t][1] = p[1];
      wsc[t] = *reinterpret_cast<const uint16_t*>(sb_ptr[t] + sbo);
    }
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) acc[i][j] = mfma_fp4<0>(wb[i][0], wsc[i], xa[j][0], xs[j], acc[i][j]);
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) acc[i][j] = mfma_fp4<1>(wb[i][1], wsc[i], xa[j][1], xs[j], acc[i][j]);
  }
  if (K % 256) {   // one 128-wide tail step, natural K order
    const size_t cb = static_cast<size_t>(k256) * 128 + grp * 16;
    const size_t sbo = static_cast<size_t>(k256) * 8 + grp;
    uint4 xa[kTM], wb[kTN];
    uint32_t xs[kTM], wsc[kTN];
#pragma unroll
    for (int t = 0; t < kTM; ++t) {
      xa[t] = *reinterpret_cast<const uint4*>(a_ptr[t] + cb);
      xs[t] = sa_ptr[t][sbo];
    }
#pragma unroll
    for (int t = 0; t < kTN; ++t) {
      wb[t] = *reinterpret_cast<const uint4*>(b_ptr[t] + cb);
      wsc[t] = sb_ptr[t][sbo];
    }
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j) acc[i][j] = mfma_fp4<0>(wb[i], wsc[i], xa[j], xs[j], acc[i][j]);
  }

  // lane holds Y[m_base + 16 j + r16][n_base + 16 i + 4 grp + 0..3]
#pragma unroll
  for (int j = 0; j < kTM; ++j) {
    const int m = m_base + 16 * j + r16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int n = n_base + 16 * i + 4 * grp;
      float* dst = Y + static_cast<size_t>(m) * N + n;
      if (n + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n + q < N) dst[q] = acc[i][j][q];
      }
    }
  }
}

}  // namespace

namespace wush {

wush_status gemm_mxfp4(int M, int N, int K, const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                       float* Y, hipStream_t stream) {
  dim3 grid((N + kBlockN - 1) / kBlockN, (M + kBlockM - 1) / kBlockM);
  if (grid.y > 65535u) return fail(WUSH_E_SHAPE, "wush_w4a4_gemm: M=%d too large", M);
  hipLaunchKernelGGL(gemm_mxfp4_direct, grid, dim3(256), 0, stream, A, SA, B, SB, Y, M, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // namespace wush
