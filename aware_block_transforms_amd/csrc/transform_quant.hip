// Transform-then-quantize kernels for gfx950: the online activation step and
// the offline weight packing of WUSH.
//
// WUSH news article (chain.bitekongjian.com), deployment paragraph: at
// inference only the activations are transformed, one small matrix per block
// of input channels; weights are transformed and quantized once, offline.
// "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization" (AI Radio),
// "The gist": transform and quantizer run as one fused GPU kernel.
//
// Work mapping (CDNA4, wave64):
//  * one wave owns one block b of channels and two tiles of 64 tokens; lane
//    l holds tokens base + l and base + 64 + l.  The block's bs x bs matrix is
//    identical for every lane, so it is read with scalar loads into SGPRs and
//    broadcast to the FMAs for free, each element serving both tokens (the
//    scalar cache's bandwidth, not the VALU, bounds a one-token loop); the
//    wave's x values stay in VGPRs.
//  * y_i = fma chain over k (ascending, from +0) in fp32: bs*bs v_fma_f32 per
//    lane and block.  All bs outputs of a block live in one lane, so the block
//    maximum needs no cross-lane reduction.
//  * the lane packs its bs codes into bs/2 contiguous bytes (one 16-byte store
//    at bs = 32) and stores one scale.
// The arithmetic is pinned (see wush.h): codes and scales are bit-exact
// functions of (T, x).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kTokensPerWave = 2 * kWave;   // two 64-token tiles per wave

enum Fmt { kMX = 0, kNV = 1, kI4 = 2, kAmax = 3 };

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E2M1 code: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, exact ties to the even
// code, saturating, sign bit copied.  Counts the decision thresholds passed.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float m = fabsf(v);
  uint32_t c = (m > 0.25f ? 1u : 0u) + (m >= 0.75f ? 1u : 0u) + (m > 1.25f ? 1u : 0u) +
               (m >= 1.75f ? 1u : 0u) + (m > 2.5f ? 1u : 0u) + (m >= 3.5f ? 1u : 0u) +
               (m > 5.0f ? 1u : 0u);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// Same, but NaN encodes as 0 (needed where v may be 0 * inf).
__device__ __forceinline__ uint32_t e2m1_code_nan0(float v) {
  return (v == v) ? e2m1_code(v) : 0u;
}

// FP8 E4M3 (finite-only) of 0 <= s <= 448, round to nearest, ties to even.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (s < 0.015625f) {                       // below 2^-6: subnormal grid m * 2^-9
    return static_cast<uint32_t>(rintf(s * 512.0f));   // 0..8 (8 = 2^-6, code 0x08)
  }
  uint32_t b = __float_as_uint(s);
  b += 0x7ffffu + ((b >> 20) & 1u);          // round to 3 mantissa bits, ties to even
  return (b >> 20) - (120u << 3);            // rebias exponent 127 -> 7
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t ex = (c >> 3) & 15u, m = c & 7u;
  if (ex == 0) return static_cast<float>(m) * 0.001953125f;   // m * 2^-9
  return __uint_as_float(((ex + 120u) << 23) | (m << 20));
}

template <int BS, bool BF16>
__device__ __forceinline__ void load_block(const void* __restrict__ X, size_t off, float (&x)[BS]) {
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(X) + off);
#pragma unroll
    for (int q = 0; q < BS / 8; ++q) {
      const uint4 w = p[q];
      x[8 * q + 0] = bf16lo(w.x); x[8 * q + 1] = bf16hi(w.x);
      x[8 * q + 2] = bf16lo(w.y); x[8 * q + 3] = bf16hi(w.y);
      x[8 * q + 4] = bf16lo(w.z); x[8 * q + 5] = bf16hi(w.z);
      x[8 * q + 6] = bf16lo(w.w); x[8 * q + 7] = bf16hi(w.w);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(X) + off);
#pragma unroll
    for (int q = 0; q < BS / 4; ++q) {
      const float4 w = p[q];
      x[4 * q + 0] = w.x; x[4 * q + 1] = w.y; x[4 * q + 2] = w.z; x[4 * q + 3] = w.w;
    }
  }
}

// y = T x for two tokens at once, each with the pinned fp32 FMA chain.  Tb is
// wave-uniform (scalar loads into SGPRs); every T element fetched through the
// scalar cache feeds two FMAs, which halves the scalar-cache traffic that
// otherwise bounds this kernel.
// Rows of T are double-buffered in SGPRs: row i+1 is requested before the
// FMAs of row i, and the fences keep the compiler from hoisting every row's
// loads (which runs out of SGPRs and spills them to VGPR lanes).
template <int BS>
__device__ __forceinline__ void transform2(const float* __restrict__ Tb, const float (&x0)[BS], const float (&x1)[BS],
                                           float (&y0)[BS], float (&y1)[BS]) {
  float tc[BS], tn[BS];
#pragma unroll
  for (int k = 0; k < BS; ++k) tc[k] = Tb[k];
#pragma unroll
  for (int i = 0; i < BS; ++i) {
    if (i + 1 < BS) {
#pragma unroll
      for (int k = 0; k < BS; ++k) tn[k] = Tb[(i + 1) * BS + k];
    }
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int k = 0; k < BS; ++k) {
      a0 = __builtin_fmaf(tc[k], x0[k], a0);
      a1 = __builtin_fmaf(tc[k], x1[k], a1);
    }
    y0[i] = a0;
    y1[i] = a1;
#pragma unroll
    for (int k = 0; k < BS; ++k) tc[k] = tn[k];
    asm volatile("" ::: "memory");   // keeps the next row's loads here at the IR level too
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Two E2M1 codes into byte `sel` of `old` (low nibble = a).  gfx950's packed FP4
// conversion rounds to nearest with ties to the even code, saturates at 6 and keeps
// the sign bit, which is exactly the pinned encoder for every non-NaN input; the
// scale operand divides, so 1.0 leaves the values unchanged.
__device__ __forceinline__ uint32_t cvt_pair(uint32_t old, float a, float b, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 3);
  }
}

template <int N>
__device__ __forceinline__ void zero_words(uint32_t (&w)[N]) {
#pragma unroll
  for (int q = 0; q < N; ++q) w[q] = 0u;
}

template <int BS>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ dst, const uint32_t (&w)[BS / 8]) {
  if constexpr (BS == 32) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  }
}

// Codes and scale of one token's block y (the pinned encoders); `amax` pass
// only folds the block maximum into run_max.
template <int BS, int FMT>
__device__ __forceinline__ void encode_store(const float (&y)[BS], size_t row, int blk, int nblk, int d_in, float g,
                                             uint8_t* __restrict__ codes, void* __restrict__ scales,
                                             uint32_t& run_max) {
  uint32_t ab = 0;
#pragma unroll
  for (int k = 0; k < BS; ++k) ab = max(ab, __float_as_uint(y[k]) & 0x7fffffffu);
  const bool bad = ab >= 0x7f800000u;          // NaN or Inf in the block
  if constexpr (FMT == kAmax) {
    run_max = max(run_max, ab);
    return;
  } else {
    uint32_t w[BS / 8];
#pragma unroll
    for (int q = 0; q < BS / 8; ++q) w[q] = 0u;
    if constexpr (FMT == kMX) {
      const uint32_t ex = ab >> 23;
      const uint32_t sbyte = ex > 2u ? ex - 2u : 0u;             // e + 127
      const float inv = __uint_as_float((254u - sbyte) << 23);   // 2^-e
#pragma unroll
      for (int k = 0; k < BS / 2; ++k) w[k >> 2] = cvt_pair(w[k >> 2], y[2 * k] * inv, y[2 * k + 1] * inv, k & 3);
      if (bad) zero_words(w);
      reinterpret_cast<uint8_t*>(scales)[row * nblk + blk] = bad ? 0xffu : static_cast<uint8_t>(sbyte);
    } else if constexpr (FMT == kNV) {
      const float a = __uint_as_float(ab);
      float s = fminf(a / (6.0f * g), 448.0f);
      const uint32_t s8 = bad ? 0u : e4m3_encode(s);
      const float s_eff = e4m3_decode(s8) * g;
      const float r = 1.0f / s_eff;
      const bool zero = bad || s_eff == 0.0f;
      if (r <= 3.0e38f) {                       // finite r: every y * r is a number
#pragma unroll
        for (int k = 0; k < BS / 2; ++k) w[k >> 2] = cvt_pair(w[k >> 2], y[2 * k] * r, y[2 * k + 1] * r, k & 3);
      } else {                                  // s_eff below 2^-128: 0 * inf is NaN -> code 0
#pragma unroll
        for (int k = 0; k < BS; ++k) w[k >> 3] |= e2m1_code_nan0(y[k] * r) << (4 * (k & 7));
      }
      if (zero) zero_words(w);
      reinterpret_cast<uint8_t*>(scales)[row * nblk + blk] = bad ? 0x7fu : static_cast<uint8_t>(s8);
    } else {  // INT4
      const float a = __uint_as_float(ab);
      const _Float16 h = static_cast<_Float16>(a / 7.0f);        // RNE
      const float s32 = static_cast<float>(h);
      const float r = 1.0f / s32;
      const bool zero = bad || s32 == 0.0f;
      // clamp to [-7, 7], then add 1.5 * 2^23: the fp32 add rounds to the nearest
      // integer (ties to even) and leaves q in the low mantissa bits (two's complement)
#pragma unroll
      for (int k = 0; k < BS; ++k) {
        const float t = __builtin_amdgcn_fmed3f(y[k] * r, -7.0f, 7.0f) + 12582912.0f;
        w[k >> 3] |= (__float_as_uint(t) & 15u) << (4 * (k & 7));
      }
      if (zero) zero_words(w);
      uint16_t hb;
      __builtin_memcpy(&hb, &h, 2);
      reinterpret_cast<uint16_t*>(scales)[row * nblk + blk] = bad ? static_cast<uint16_t>(0x7e00u) : hb;
    }
    store_codes<BS>(codes + row * (d_in / 2) + static_cast<size_t>(blk) * (BS / 2), w);
  }
}

// One kernel for the three formats plus an amax-only pass (NVFP4 tensor scale).
// A wave owns one block and two 64-token tiles: lane l transforms tokens
// base + l and base + 64 + l together (see transform2).
template <int BS, int FMT, bool BF16, bool IDENT>
__global__ __launch_bounds__(kWave * kWavesPerGroup) __attribute__((amdgpu_waves_per_eu(4))) void tq_kernel(
    const void* __restrict__ X, const float* __restrict__ T, int n, int d_in, float g,
    uint8_t* __restrict__ codes, void* __restrict__ scales, uint32_t* __restrict__ amax_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = d_in / BS;
  const int blk = blockIdx.x * kWavesPerGroup + wave;
  if (blk >= nblk) return;                       // wave-uniform
  const float* __restrict__ Tb = IDENT ? nullptr : T + static_cast<size_t>(blk) * BS * BS;
  const int tok0 = blockIdx.y * (2 * kWave) + lane, tok1 = tok0 + kWave;
  const bool v0 = tok0 < n, v1 = tok1 < n;
  uint32_t run_max = 0;

  float x0[BS], x1[BS];
  const size_t col = static_cast<size_t>(blk) * BS;
  if (v0) load_block<BS, BF16>(X, static_cast<size_t>(tok0) * d_in + col, x0);
  if (v1) load_block<BS, BF16>(X, static_cast<size_t>(tok1) * d_in + col, x1);
  else {
#pragma unroll
    for (int k = 0; k < BS; ++k) x1[k] = 0.0f;
  }

  float y0[BS], y1[BS];
  if constexpr (IDENT) {
#pragma unroll
    for (int k = 0; k < BS; ++k) { y0[k] = x0[k]; y1[k] = x1[k]; }
  } else {
    transform2<BS>(Tb, x0, x1, y0, y1);
    // materialize both tokens' outputs here: left alone, the compiler sinks
    // each token's FMAs into its (divergent) store branch, and the T values
    // both branches share then pile up in SGPRs
#pragma unroll
    for (int k = 0; k < BS; ++k) asm volatile("" : "+v"(y0[k]), "+v"(y1[k]));
  }
  if (v0) encode_store<BS, FMT>(y0, static_cast<size_t>(tok0), blk, nblk, d_in, g, codes, scales, run_max);
  if (v1) encode_store<BS, FMT>(y1, static_cast<size_t>(tok1), blk, nblk, d_in, g, codes, scales, run_max);

  if constexpr (FMT == kAmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) run_max = max(run_max, static_cast<uint32_t>(__shfl_xor(static_cast<int>(run_max), off)));
    if (lane == 0) atomicMax(amax_out, run_max);
  }
}

// Hadamard-diagonal variant (news article, deployment and limitation
// paragraphs: the data-aware component approximated by a diagonal matrix):
// y = H_bs (d o x) per block, pinned as one fp32 product per element and then
// butterfly stages h = 1, 2, ..., bs/2 (no fused multiply-add).  With bs + 5
// operations per element instead of 2 bs, the step is bound by HBM, so the
// mapping is chosen for the memory stream: one lane per (token, block), the
// lanes of a wave on 64 consecutive blocks of one token row (contiguous 64 B
// per lane, 4 KB per wave at bs 32 and bf16), each wave on kHdTokens tokens,
// whose loads are all issued before the first is used.  The lane's d values
// stay in VGPRs.
constexpr int kHdTokens = 2;

template <int BS>
__device__ __forceinline__ void hd_rotate(float (&v)[BS]) {
#pragma unroll
  for (int h = 1; h < BS; h <<= 1) {
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      if (j & h) continue;
      const float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
}

template <int BS, int FMT, bool BF16>
__global__ __launch_bounds__(kWave * kWavesPerGroup) void tq_hd_kernel(
    const void* __restrict__ X, const float* __restrict__ d, int n, int d_in, float g,
    uint8_t* __restrict__ codes, void* __restrict__ scales, uint32_t* __restrict__ amax_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = d_in / BS;
  const int blk = blockIdx.x * kWave + lane;
  const bool vb = blk < nblk;
  const int tok0 = (blockIdx.y * kWavesPerGroup + wave) * kHdTokens;
  // Loads are unconditional (a conditional load makes every later wait a full
  // drain): lanes past the last block and tokens past n re-read the last one,
  // and only the stores below are guarded.
  const size_t col = static_cast<size_t>(min(blk, nblk - 1)) * BS;
  uint32_t run_max = 0;
  float x[kHdTokens][BS];
#pragma unroll
  for (int t = 0; t < kHdTokens; ++t)
    load_block<BS, BF16>(X, static_cast<size_t>(min(tok0 + t, n - 1)) * d_in + col, x[t]);
  float dv[BS];
  {
    const float4* p = reinterpret_cast<const float4*>(d + col);
#pragma unroll
    for (int q = 0; q < BS / 4; ++q) {
      const float4 w = p[q];
      dv[4 * q + 0] = w.x; dv[4 * q + 1] = w.y; dv[4 * q + 2] = w.z; dv[4 * q + 3] = w.w;
    }
  }
#pragma unroll
  for (int t = 0; t < kHdTokens; ++t) {
    if (vb && tok0 + t < n) {
#pragma unroll
      for (int k = 0; k < BS; ++k) x[t][k] = x[t][k] * dv[k];
      hd_rotate<BS>(x[t]);
      encode_store<BS, FMT>(x[t], static_cast<size_t>(tok0 + t), blk, nblk, d_in, g, codes, scales, run_max);
    }
  }
  if constexpr (FMT == kAmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) run_max = max(run_max, static_cast<uint32_t>(__shfl_xor(static_cast<int>(run_max), off)));
    if (lane == 0) atomicMax(amax_out, run_max);
  }
}

__global__ void fill_u32(uint32_t* p, uint32_t v) { *p = v; }

using KernelFn = void (*)(const void*, const float*, int, int, float, uint8_t*, void*, uint32_t*);

template <int BS, int FMT>
KernelFn pick(bool bf16, bool ident) {
  if (bf16) return ident ? tq_kernel<BS, FMT, true, true> : tq_kernel<BS, FMT, true, false>;
  return ident ? tq_kernel<BS, FMT, false, true> : tq_kernel<BS, FMT, false, false>;
}

KernelFn select_kernel(int fmt, int bs, bool bf16, bool ident) {
  if (bs == 32) {
    switch (fmt) {
      case kMX: return pick<32, kMX>(bf16, ident);
      case kI4: return pick<32, kI4>(bf16, ident);
      case kAmax: return pick<32, kAmax>(bf16, ident);
    }
  } else if (bs == 16) {
    switch (fmt) {
      case kNV: return pick<16, kNV>(bf16, ident);
      case kAmax: return pick<16, kAmax>(bf16, ident);
    }
  }
  return nullptr;
}

wush_status launch(int fmt, int bs, bool bf16, int n, int d_in, const void* X, const float* T, float g,
                   uint8_t* codes, void* scales, uint32_t* amax, hipStream_t stream) {
  if (n == 0) return WUSH_OK;
  KernelFn k = select_kernel(fmt, bs, bf16, T == nullptr);
  if (!k) return wush::fail(WUSH_E_UNSUPPORTED, "transform_quant: no kernel for fmt=%d bs=%d", fmt, bs);
  const int nblk = d_in / bs;
  dim3 grid((nblk + kWavesPerGroup - 1) / kWavesPerGroup, (n + kTokensPerWave - 1) / kTokensPerWave);
  if (grid.y > 65535u) return wush::fail(WUSH_E_SHAPE, "transform_quant: n=%d too large", n);
  hipLaunchKernelGGL(k, grid, dim3(kWave * kWavesPerGroup), 0, stream, X, T, n, d_in, g, codes, scales, amax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "transform_quant launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

KernelFn select_hd_kernel(int fmt, int bs, bool bf16) {
  if (bs == 32) {
    switch (fmt) {
      case kMX: return bf16 ? tq_hd_kernel<32, kMX, true> : tq_hd_kernel<32, kMX, false>;
      case kI4: return bf16 ? tq_hd_kernel<32, kI4, true> : tq_hd_kernel<32, kI4, false>;
      case kAmax: return bf16 ? tq_hd_kernel<32, kAmax, true> : tq_hd_kernel<32, kAmax, false>;
    }
  } else if (bs == 16) {
    switch (fmt) {
      case kNV: return bf16 ? tq_hd_kernel<16, kNV, true> : tq_hd_kernel<16, kNV, false>;
      case kAmax: return bf16 ? tq_hd_kernel<16, kAmax, true> : tq_hd_kernel<16, kAmax, false>;
    }
  }
  return nullptr;
}

wush_status launch_hd(int fmt, int bs, bool bf16, int n, int d_in, const void* X, const float* d, float g,
                      uint8_t* codes, void* scales, uint32_t* amax, hipStream_t stream) {
  if (n == 0) return WUSH_OK;
  KernelFn k = select_hd_kernel(fmt, bs, bf16);
  if (!k) return wush::fail(WUSH_E_UNSUPPORTED, "transform_quant_hd: no kernel for fmt=%d bs=%d", fmt, bs);
  const int nblk = d_in / bs;
  const int per_group = kWavesPerGroup * kHdTokens;
  dim3 grid((nblk + kWave - 1) / kWave, (n + per_group - 1) / per_group);
  if (grid.y > 65535u) return wush::fail(WUSH_E_SHAPE, "transform_quant_hd: n=%d too large", n);
  hipLaunchKernelGGL(k, grid, dim3(kWave * kWavesPerGroup), 0, stream, X, d, n, d_in, g, codes, scales, amax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "transform_quant_hd launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

// max|T x| over a tensor, written to a device uint (float bits).
// (T is a dense [nblk][bs][bs] matrix, or with hd the per-channel scales.)
wush_status tensor_amax(int bs, bool bf16, int n, int d_in, const void* X, const float* T, bool hd,
                        uint32_t* amax_dev, hipStream_t stream) {
  hipLaunchKernelGGL(fill_u32, dim3(1), dim3(1), 0, stream, amax_dev, 0u);
  if (hd) return launch_hd(kAmax, bs, bf16, n, d_in, X, T, 0.0f, nullptr, nullptr, amax_dev, stream);
  return launch(kAmax, bs, bf16, n, d_in, X, T, 0.0f, nullptr, nullptr, amax_dev, stream);
}

wush_status global_scale(int bs, bool bf16, int n, int d_in, const void* X, const float* T, bool hd, float* g_out,
                         hipStream_t stream) {
  uint32_t* dbuf = nullptr;
  if (hipMalloc(&dbuf, sizeof(uint32_t)) != hipSuccess) return wush::fail(WUSH_E_HIP, "global_scale: hipMalloc failed");
  wush_status st = tensor_amax(bs, bf16, n, d_in, X, T, hd, dbuf, stream);
  uint32_t bits = 0;
  if (st == WUSH_OK) {
    if (hipMemcpyAsync(&bits, dbuf, sizeof bits, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      st = wush::fail(WUSH_E_HIP, "global_scale: copy back failed");
  }
  (void)hipFree(dbuf);
  if (st != WUSH_OK) return st;
  float amax;
  __builtin_memcpy(&amax, &bits, 4);
  if (!(amax > 0.0f) || bits >= 0x7f800000u)
    return wush::fail(WUSH_E_NUMERIC, "global_scale: tensor maximum is zero or not finite");
  *g_out = amax / 2688.0f;   // 6 * 448
  return WUSH_OK;
}

wush_status check_common(const char* who, wush_format fmt, int rows, int d_in, const void* X, uint8_t* codes,
                         void* scales) {
  const int bs = wush_format_block(fmt);
  if (bs == 0) return wush::fail(WUSH_E_ARG, "%s: bad format %d", who, static_cast<int>(fmt));
  if (rows < 0 || d_in < bs || d_in % bs != 0)
    return wush::fail(WUSH_E_SHAPE, "%s: need rows >= 0 and d_in a positive multiple of %d (rows=%d d_in=%d)", who,
                      bs, rows, d_in);
  if (rows > 0 && (!X || !codes || !scales)) return wush::fail(WUSH_E_ARG, "%s: null pointer", who);
  if (!wush::aligned16(X) || !wush::aligned16(codes))
    return wush::fail(WUSH_E_ARG, "%s: X and codes must be 16-byte aligned", who);
  return WUSH_OK;
}

}  // namespace

extern "C" {

wush_status wush_transform_quant(wush_format fmt, wush_dtype xdt, int n, int d_in, const void* X, const float* Tx,
                                 float g, uint8_t* codes, void* scales, void* stream) {
  wush_status st = check_common("wush_transform_quant", fmt, n, d_in, X, codes, scales);
  if (st != WUSH_OK) return st;
  if (xdt != WUSH_F32 && xdt != WUSH_BF16) return wush::fail(WUSH_E_ARG, "wush_transform_quant: bad dtype");
  if (fmt == WUSH_NVFP4 && !(g > 0.0f && g < 3.0e38f))
    return wush::fail(WUSH_E_ARG, "wush_transform_quant: NVFP4 needs a positive finite tensor scale g");
  const int fk = fmt == WUSH_MXFP4 ? kMX : fmt == WUSH_NVFP4 ? kNV : kI4;
  return launch(fk, wush_format_block(fmt), xdt == WUSH_BF16, n, d_in, X, Tx, g, codes, scales, nullptr,
                static_cast<hipStream_t>(stream));
}

wush_status wush_nvfp4_global_scale(wush_dtype xdt, int n, int d_in, const void* X, const float* Tx, float* g_out,
                                    void* stream) {
  if (!X || !g_out) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale: null pointer");
  if (xdt != WUSH_F32 && xdt != WUSH_BF16) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale: bad dtype");
  if (n < 1 || d_in < 16 || d_in % 16 != 0)
    return wush::fail(WUSH_E_SHAPE, "wush_nvfp4_global_scale: need n >= 1 and d_in %% 16 == 0");
  if (!wush::aligned16(X)) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale: X must be 16-byte aligned");
  return global_scale(16, xdt == WUSH_BF16, n, d_in, X, Tx, false, g_out, static_cast<hipStream_t>(stream));
}

wush_status wush_pack_weights(wush_format fmt, int d_out, int d_in, const float* W, const float* Tw, uint8_t* codes,
                              void* scales, float* g_out, void* stream) {
  wush_status st = check_common("wush_pack_weights", fmt, d_out, d_in, W, codes, scales);
  if (st != WUSH_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float g = 0.0f;
  if (fmt == WUSH_NVFP4) {
    if (!g_out) return wush::fail(WUSH_E_ARG, "wush_pack_weights: NVFP4 needs g_out");
    if (d_out < 1) return wush::fail(WUSH_E_SHAPE, "wush_pack_weights: NVFP4 needs d_out >= 1");
    st = global_scale(16, false, d_out, d_in, W, Tw, false, &g, s);
    if (st != WUSH_OK) return st;
    *g_out = g;
  } else if (g_out) {
    *g_out = 1.0f;
  }
  const int fk = fmt == WUSH_MXFP4 ? kMX : fmt == WUSH_NVFP4 ? kNV : kI4;
  return launch(fk, wush_format_block(fmt), false, d_out, d_in, W, Tw, g, codes, scales, nullptr, s);
}

wush_status wush_transform_quant_hd(wush_format fmt, wush_dtype xdt, int n, int d_in, const void* X, const float* dx,
                                    float g, uint8_t* codes, void* scales, void* stream) {
  wush_status st = check_common("wush_transform_quant_hd", fmt, n, d_in, X, codes, scales);
  if (st != WUSH_OK) return st;
  if (xdt != WUSH_F32 && xdt != WUSH_BF16) return wush::fail(WUSH_E_ARG, "wush_transform_quant_hd: bad dtype");
  if (n > 0 && !dx) return wush::fail(WUSH_E_ARG, "wush_transform_quant_hd: null scales d");
  if (!wush::aligned16(dx)) return wush::fail(WUSH_E_ARG, "wush_transform_quant_hd: d must be 16-byte aligned");
  if (fmt == WUSH_NVFP4 && !(g > 0.0f && g < 3.0e38f))
    return wush::fail(WUSH_E_ARG, "wush_transform_quant_hd: NVFP4 needs a positive finite tensor scale g");
  const int fk = fmt == WUSH_MXFP4 ? kMX : fmt == WUSH_NVFP4 ? kNV : kI4;
  return launch_hd(fk, wush_format_block(fmt), xdt == WUSH_BF16, n, d_in, X, dx, g, codes, scales, nullptr,
                   static_cast<hipStream_t>(stream));
}

wush_status wush_nvfp4_global_scale_hd(wush_dtype xdt, int n, int d_in, const void* X, const float* dx, float* g_out,
                                       void* stream) {
  if (!X || !dx || !g_out) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale_hd: null pointer");
  if (xdt != WUSH_F32 && xdt != WUSH_BF16) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale_hd: bad dtype");
  if (n < 1 || d_in < 16 || d_in % 16 != 0)
    return wush::fail(WUSH_E_SHAPE, "wush_nvfp4_global_scale_hd: need n >= 1 and d_in %% 16 == 0");
  if (!wush::aligned16(X) || !wush::aligned16(dx))
    return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale_hd: X and d must be 16-byte aligned");
  return global_scale(16, xdt == WUSH_BF16, n, d_in, X, dx, true, g_out, static_cast<hipStream_t>(stream));
}

wush_status wush_pack_weights_hd(wush_format fmt, int d_out, int d_in, const float* W, const float* dw, uint8_t* codes,
                                 void* scales, float* g_out, void* stream) {
  wush_status st = check_common("wush_pack_weights_hd", fmt, d_out, d_in, W, codes, scales);
  if (st != WUSH_OK) return st;
  if (d_out > 0 && !dw) return wush::fail(WUSH_E_ARG, "wush_pack_weights_hd: null scales d");
  if (!wush::aligned16(dw)) return wush::fail(WUSH_E_ARG, "wush_pack_weights_hd: d must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float g = 0.0f;
  if (fmt == WUSH_NVFP4) {
    if (!g_out) return wush::fail(WUSH_E_ARG, "wush_pack_weights_hd: NVFP4 needs g_out");
    if (d_out < 1) return wush::fail(WUSH_E_SHAPE, "wush_pack_weights_hd: NVFP4 needs d_out >= 1");
    st = global_scale(16, false, d_out, d_in, W, dw, true, &g, s);
    if (st != WUSH_OK) return st;
    *g_out = g;
  } else if (g_out) {
    *g_out = 1.0f;
  }
  const int fk = fmt == WUSH_MXFP4 ? kMX : fmt == WUSH_NVFP4 ? kNV : kI4;
  return launch_hd(fk, wush_format_block(fmt), false, d_out, d_in, W, dw, g, codes, scales, nullptr, s);
}

}  // extern "C"
