// Hadamard-256 pre-rotated 3-bit weights and the matching GEMV for gfx950.
//
// ITQ3_S article (ai.866data.com), section on the core technique: each
// 256-element weight vector is rotated by a fast Walsh-Hadamard transform so
// that outlier energy spreads over the vector, then quantized with a uniform
// 3-bit grid; at inference the inverse rotation is folded into the load path
// and the rotate / inverse-rotate round trip is exact.
//
// Pack: one workgroup of 256 threads per 256-vector; the 8 butterfly stages
// run through LDS in the pinned order (h = 1, 2, ..., 128), then x 1/16, the
// vector maximum, an fp16 scale and codes in [-3, 3] stored as two bit planes.
//
// GEMV: instead of inverse-rotating every weight (8 butterflies per weight on
// the vector ALU), the rotation is moved to the activations, which every
// output row shares:  sum_k x_k * (s/16)(H q)_k = (s/16) * sum_m q_m (H x)_m
// because H is symmetric.  Each workgroup rotates the activation chunks it
// needs in LDS once and then streams the packed weights, so the weight path
// does only unpack + multiply-add.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

constexpr int kVec = 256;
constexpr int kBytes = 96;
constexpr int kRows = 64;      // output rows per GEMV workgroup (one per lane)
constexpr int kChunks = 4;     // 256-chunks rotated per phase (one per wave)

// In-place forward FWHT of a 256-vector held one element per thread in `v`
// (LDS).  Thread t returns its element after all 8 stages.
__device__ __forceinline__ float fwht256_lds(float* v, float val) {
  const int t = threadIdx.x;
  v[t] = val;
  __syncthreads();
#pragma unroll
  for (int h = 1; h < kVec; h <<= 1) {
    const float mine = v[t];
    const float other = v[t ^ h];
    __syncthreads();
    const float nv = (t & h) ? (other - mine) : (mine + other);
    v[t] = nv;
    __syncthreads();
  }
  return v[t];
}

__global__ __launch_bounds__(kVec) void had256_pack_kernel(const float* __restrict__ W, int d_in,
                                                           uint8_t* __restrict__ planes,
                                                           uint16_t* __restrict__ scales) {
  __shared__ float v[kVec];
  __shared__ uint32_t wmax[kVec / 64];
  __shared__ uint8_t cc[kVec];
  const int t = threadIdx.x;
  const int nv = d_in / kVec;
  const size_t vec = blockIdx.x;                 // row * nv + chunk
  const size_t row = vec / nv, c = vec % nv;
  const float x = W[row * d_in + c * kVec + t];
  const float r0 = fwht256_lds(v, x) * 0.0625f;
  uint32_t ab = __float_as_uint(r0) & 0x7fffffffu;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ab = max(ab, static_cast<uint32_t>(__shfl_xor(static_cast<int>(ab), off)));
  if ((t & 63) == 0) wmax[t >> 6] = ab;
  __syncthreads();
  ab = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float a = __uint_as_float(ab);
  const _Float16 h = static_cast<_Float16>(a / 3.0f);
  const float s32 = static_cast<float>(h);
  int q = 0;
  if (s32 != 0.0f) {
    const float r = 1.0f / s32;
    q = static_cast<int>(fminf(fmaxf(rintf(r0 * r), -3.0f), 3.0f));
  }
  cc[t] = static_cast<uint8_t>(q & 7);
  __syncthreads();
  uint8_t* dst = planes + vec * kBytes;
  if (t < 64) {
    dst[t] = static_cast<uint8_t>((cc[4 * t] & 3) | ((cc[4 * t + 1] & 3) << 2) | ((cc[4 * t + 2] & 3) << 4) |
                                  ((cc[4 * t + 3] & 3) << 6));
  } else if (t < 96) {
    const int j = t - 64;
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) b |= ((cc[8 * j + i] >> 2) & 1u) << i;
    dst[t] = static_cast<uint8_t>(b);
  }
  if (t == 0) {
    uint16_t hb;
    __builtin_memcpy(&hb, &h, 2);
    scales[vec] = hb;
  }
}

__global__ __launch_bounds__(kVec) void had256_rotate_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                             int d_in) {
  __shared__ float v[kVec];
  const int t = threadIdx.x;
  const int nv = d_in / kVec;
  const size_t vec = blockIdx.x;
  const size_t off = (vec / nv) * d_in + (vec % nv) * kVec + t;
  const float x = in[off];
  const float r = fwht256_lds(v, x) * 0.0625f;
  out[off] = r;
}

// Signed 3-bit code m of a packed 96-byte vector whose two planes are in
// registers: lo = bytes 0..63 as 16 dwords, hi = bytes 64..95 as 8 dwords.
__device__ __forceinline__ float code_at(const uint32_t (&lo)[16], const uint32_t (&hi)[8], int m) {
  const uint32_t l2 = (lo[m >> 4] >> (2 * (m & 15))) & 3u;
  const uint32_t b2 = (hi[m >> 5] >> (m & 31)) & 1u;
  const int c = static_cast<int>(l2 | (b2 << 2));
  return static_cast<float>((c ^ 4) - 4);
}

template <int B>
__global__ __launch_bounds__(256) void had256_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const uint8_t* __restrict__ planes,
                                                          const uint16_t* __restrict__ scales,
                                                          float* __restrict__ y, int nb, int d_out, int d_in) {
  // B is the compiled batch capacity; nb <= B rows of x / y are real.
  __shared__ float xs[B * kChunks * kVec];   // rotated activations, [b][chunk][256]
  __shared__ float red[kChunks * B * kRows];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nv = d_in / kVec;
  const int row = blockIdx.x * kRows + lane;
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;

  for (int p = 0; p < nv; p += kChunks) {
    __syncthreads();
    for (int i = t; i < B * kChunks * kVec; i += 256) {
      const int b = i / (kChunks * kVec), j = i % (kChunks * kVec);
      const int c = p + j / kVec;
      xs[i] = (c < nv && b < nb) ? __uint_as_float(static_cast<uint32_t>(x[static_cast<size_t>(b) * d_in + p * kVec + j]) << 16)
                     : 0.0f;
    }
    __syncthreads();
    // unnormalised H x for every (b, chunk) vector: 8 butterfly stages
    for (int h = 1; h < kVec; h <<= 1) {
      for (int i = t; i < B * kChunks * (kVec / 2); i += 256) {
        const int vid = i / (kVec / 2), pi = i % (kVec / 2);
        const int lo = (pi / h) * 2 * h + (pi % h);
        float* base = xs + vid * kVec;
        const float a = base[lo], bb = base[lo + h];
        base[lo] = a + bb;
        base[lo + h] = a - bb;
      }
      __syncthreads();
    }
    const int c = p + wave;
    if (c < nv && row < d_out) {
      const size_t vec = static_cast<size_t>(row) * nv + c;
      const uint4* wp = reinterpret_cast<const uint4*>(planes + vec * kBytes);
      uint32_t lo[16], hi[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w = wp[q];
        lo[4 * q] = w.x; lo[4 * q + 1] = w.y; lo[4 * q + 2] = w.z; lo[4 * q + 3] = w.w;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 w = wp[4 + q];
        hi[4 * q] = w.x; hi[4 * q + 1] = w.y; hi[4 * q + 2] = w.z; hi[4 * q + 3] = w.w;
      }
      const uint16_t sb = scales[vec];
      _Float16 hs;
      __builtin_memcpy(&hs, &sb, 2);
      const float s = static_cast<float>(hs) * 0.0625f;
      float part[B];
#pragma unroll
      for (int b = 0; b < B; ++b) part[b] = 0.0f;
      const float* xr = xs + wave * kVec;
#pragma unroll
      for (int m = 0; m < kVec; ++m) {     // fully unrolled: register-array indexes stay static
        const float q = code_at(lo, hi, m);
#pragma unroll
        for (int b = 0; b < B; ++b) part[b] = fmaf(q, xr[b * kChunks * kVec + m], part[b]);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = fmaf(s, part[b], acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < B; ++b) red[(wave * B + b) * kRows + lane] = acc[b];
  __syncthreads();
  if (wave == 0 && row < d_out) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (b >= nb) break;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kChunks; ++w) s += red[(w * B + b) * kRows + lane];
      y[static_cast<size_t>(b) * d_out + row] = s;
    }
  }
}

template <int B>
void launch_gemv(int nb, int d_out, int d_in, const uint16_t* x, const uint8_t* planes, const uint16_t* scales, float* y,
                 hipStream_t s) {
  hipLaunchKernelGGL(had256_gemv_kernel<B>, dim3((d_out + kRows - 1) / kRows), dim3(256), 0, s, x, planes, scales, y,
                     nb, d_out, d_in);
}

}  // namespace

extern "C" {

wush_status wush_had256_pack_weights(int d_out, int d_in, const float* W, uint8_t* planes, uint16_t* scales,
                                     void* stream) {
  if (d_out < 0 || d_in < kVec || d_in % kVec)
    return wush::fail(WUSH_E_SHAPE, "wush_had256_pack_weights: d_in must be a positive multiple of 256");
  if (d_out == 0) return WUSH_OK;
  if (!W || !planes || !scales) return wush::fail(WUSH_E_ARG, "wush_had256_pack_weights: null pointer");
  const size_t nvec = static_cast<size_t>(d_out) * (d_in / kVec);
  if (nvec > 0x7fffffffu) return wush::fail(WUSH_E_SHAPE, "wush_had256_pack_weights: too many vectors");
  hipLaunchKernelGGL(had256_pack_kernel, dim3(static_cast<unsigned>(nvec)), dim3(kVec), 0,
                     static_cast<hipStream_t>(stream), W, d_in, planes, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_pack_weights launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_had256_rotate(int rows, int d_in, const float* in, float* out, void* stream) {
  if (rows < 0 || d_in < kVec || d_in % kVec)
    return wush::fail(WUSH_E_SHAPE, "wush_had256_rotate: d_in must be a positive multiple of 256");
  if (rows == 0) return WUSH_OK;
  if (!in || !out) return wush::fail(WUSH_E_ARG, "wush_had256_rotate: null pointer");
  const size_t nvec = static_cast<size_t>(rows) * (d_in / kVec);
  if (nvec > 0x7fffffffu) return wush::fail(WUSH_E_SHAPE, "wush_had256_rotate: too many vectors");
  hipLaunchKernelGGL(had256_rotate_kernel, dim3(static_cast<unsigned>(nvec)), dim3(kVec), 0,
                     static_cast<hipStream_t>(stream), in, out, d_in);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_rotate launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status wush_had256_gemv(int batch, int d_out, int d_in, const uint16_t* x, const uint8_t* planes,
                             const uint16_t* scales, float* y, void* stream) {
  if (batch < 1 || batch > 16 || d_out < 1 || d_in < kVec || d_in % kVec)
    return wush::fail(WUSH_E_SHAPE, "wush_had256_gemv: need 1 <= batch <= 16, d_out >= 1, d_in %% 256 == 0");
  if (!x || !planes || !scales || !y) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: null pointer");
  if (!wush::aligned16(planes)) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: planes must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 1)
    launch_gemv<1>(batch, d_out, d_in, x, planes, scales, y, s);
  else if (batch <= 4)
    launch_gemv<4>(batch, d_out, d_in, x, planes, scales, y, s);
  else
    launch_gemv<16>(batch, d_out, d_in, x, planes, scales, y, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_gemv launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // extern "C"
