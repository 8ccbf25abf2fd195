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

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kTokensPerWave = 2 * kWave;   // two 64-token tiles per wave

// kApply: write y itself (fp32); kMXP: MXFP4 with the scales written in the
// plane order of the MXFP4 matmul's LDS stage (see mxfp4_plane_offset)
enum Fmt { kMX = 0, kNV = 1, kI4 = 2, kAmax = 3, kApply = 4, kMXP = 5 };

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

template <int BS>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ dst, const uint32_t (&w)[BS / 8]) {
  if constexpr (BS == 32) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  }
}

// The pinned block quantizers, split into the block's scale (from the bit
// pattern ab of its largest |y|, which also flags NaN and Inf) and the codes
// of value pairs under that scale.
template <int FMT>
struct BlockQuant {
  float mul;        // multiplier applied to each value before encoding
  uint32_t scale;   // scale byte (E8M0, E4M3) or fp16 bits (INT4)
  bool zero;        // codes forced to 0
  bool soft;        // NVFP4 with 1/s not finite: the software encoder (0 * inf is NaN -> code 0)
};

template <int FMT>
__device__ __forceinline__ BlockQuant<FMT> block_quant(uint32_t ab, float g) {
  BlockQuant<FMT> q{1.0f, 0u, false, false};
  const bool bad = ab >= 0x7f800000u;          // NaN or Inf in the block
  if constexpr (FMT == kMX) {
    const uint32_t ex = ab >> 23;
    const uint32_t sbyte = ex > 2u ? ex - 2u : 0u;             // e + 127
    q.mul = __uint_as_float((254u - sbyte) << 23);             // 2^-e
    q.zero = bad;
    q.scale = bad ? 0xffu : sbyte;
  } else if constexpr (FMT == kNV) {
    const float a = __uint_as_float(ab);
    const float s = fminf(a / (6.0f * g), 448.0f);
    const uint32_t s8 = bad ? 0u : e4m3_encode(s);
    const float s_eff = e4m3_decode(s8) * g;
    q.mul = 1.0f / s_eff;
    q.zero = bad || s_eff == 0.0f;
    q.soft = !(q.mul <= 3.0e38f);
    q.scale = bad ? 0x7fu : s8;
  } else if constexpr (FMT == kI4) {
    const float a = __uint_as_float(ab);
    const _Float16 h = static_cast<_Float16>(a / 7.0f);        // RNE
    const float s32 = static_cast<float>(h);
    q.mul = 1.0f / s32;
    q.zero = bad || s32 == 0.0f;
    uint16_t hb;
    __builtin_memcpy(&hb, &h, 2);
    q.scale = bad ? 0x7e00u : hb;
  }
  return q;
}

// Codes of NP value pairs: pair p (values 2p, 2p+1, low nibble first) into
// byte p % 4 of w[p / 4].
template <int FMT, int NP>
__device__ __forceinline__ void encode_pairs(const float (&y)[2 * NP], const BlockQuant<FMT>& q,
                                             uint32_t (&w)[(NP + 3) / 4]) {
#pragma unroll
  for (int i = 0; i < (NP + 3) / 4; ++i) w[i] = 0u;
  if constexpr (FMT == kI4) {
    // clamp to [-7, 7], then add 1.5 * 2^23: the fp32 add rounds to the nearest
    // integer (ties to even) and leaves q in the low mantissa bits (two's complement)
#pragma unroll
    for (int k = 0; k < 2 * NP; ++k) {
      const float t = __builtin_amdgcn_fmed3f(y[k] * q.mul, -7.0f, 7.0f) + 12582912.0f;
      w[k >> 3] |= (__float_as_uint(t) & 15u) << (4 * (k & 7));
    }
  } else {
    bool soft = false;
    if constexpr (FMT == kNV) soft = q.soft;
    if (!soft) {
#pragma unroll
      for (int p = 0; p < NP; ++p) w[p >> 2] = cvt_pair(w[p >> 2], y[2 * p] * q.mul, y[2 * p + 1] * q.mul, p & 3);
    } else {
#pragma unroll
      for (int k = 0; k < 2 * NP; ++k) w[k >> 3] |= e2m1_code_nan0(y[k] * q.mul) << (4 * (k & 7));
    }
  }
  if (q.zero) {
#pragma unroll
    for (int i = 0; i < (NP + 3) / 4; ++i) w[i] = 0u;
  }
}

template <int FMT>
__device__ __forceinline__ void store_scale(void* __restrict__ scales, size_t idx, uint32_t s) {
  if constexpr (FMT == kI4)
    reinterpret_cast<uint16_t*>(scales)[idx] = static_cast<uint16_t>(s);
  else
    reinterpret_cast<uint8_t*>(scales)[idx] = static_cast<uint8_t>(s);
}

// Byte offset of the E8M0 scale of (row, 32-wide group gi) in the plane order
// the MXFP4 matmul stages through LDS (its scales_to_planes pre-pass writes the
// same layout): 2 KB per (256-row tile t, 256-wide K block kb) at
// (t nb + kb) * 2048, plane b = gi % 8 at 256 b, lane row rr = r % 16 at 16 rr,
// tile position 8 (r / 128) + (r / 16) % 8, rotated by 8 bytes in odd planes
// (r = row % 256; nb = K / 256).
__device__ __forceinline__ size_t mxfp4_plane_offset(int row, int gi, int nb) {
  const int t = row >> 8, r = row & 255, kb = gi >> 3, b = gi & 7;
  const int pos = (8 * (r >> 7) + ((r >> 4) & 7)) ^ (8 * (b & 1));
  return (static_cast<size_t>(t) * nb + kb) * 2048 + b * 256 + (r & 15) * 16 + pos;
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
  if constexpr (FMT == kAmax) {
    run_max = max(run_max, ab);
    return;
  } else {
    const BlockQuant<FMT> q = block_quant<FMT>(ab, g);
    uint32_t w[BS / 8];
    encode_pairs<FMT, BS / 2>(y, q, w);
    store_scale<FMT>(scales, row * nblk + blk, q.scale);
    store_codes<BS>(codes + row * (d_in / 2) + static_cast<size_t>(blk) * (BS / 2), w);
  }
}

// One kernel for the three formats plus an amax-only pass (NVFP4 tensor scale).
// A wave owns one block and two 64-token tiles: lane l transforms tokens
// base + l and base + 64 + l together (see transform2).
template <int BS, int FMT, bool BF16, bool IDENT>
__global__ __launch_bounds__(kWave * kWavesPerGroup) __attribute__((amdgpu_waves_per_eu(4))) void tq_kernel(
    const void* __restrict__ X, const float* __restrict__ T, int n, int d_in, float g,
    uint8_t* __restrict__ codes, void* __restrict__ scales, uint32_t* __restrict__ amax_out,
    const int* __restrict__ tmap, int ngroups) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = d_in / BS;
  const int blk = blockIdx.x * kWavesPerGroup + wave;
  if (blk >= nblk) return;                       // wave-uniform
  // the block's matrix, or with a group map its group's (ids clamped to the table)
  const int tsel = tmap ? min(max(tmap[blk], 0), ngroups - 1) : blk;
  const float* __restrict__ Tb = IDENT ? nullptr : T + static_cast<size_t>(tsel) * BS * BS;
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

// ---------------------------------------------------------------------------
// Dense transforms on the fp32 matrix cores (every non-identity T).
//
// v_mfma_f32_16x16x4_f32 adds its four products to the accumulator one at a
// time, in the order of the lane groups that supply them, each as a fused
// multiply-add with one rounding and with subnormals kept.  A chain of these
// over k = 0 .. bs-1 starting from +0 is therefore exactly the pinned FMA
// chain.  (A GPU probe compared 2.1 million 32-step chains against the
// sequential fmaf chain, with uniform, wide-exponent, subnormal, bf16-valued
// and cancelling operands, and found no difference; a model with one rounding
// per four products differed in 22-74% of them.)  The matrix cores do 64 fp32
// flop per clock per SIMD, twice the vector FMA rate, and leave the vector ALU
// to the encoders.
//
// Mapping: a wave owns one channel block and a run of tokens.  For one group
// of 16 tokens, output rows 16h .. 16h+15 of T form the 16 x 16 product
// T[16h.., :] * X_group^T, computed as bs/4 MFMAs: lane (g = l / 16, j = l % 16)
// supplies T[16h + j][4c + g] and x[token j][4c + g] to step c and ends with
// y[token j][16h + 4g + e] in register e.
//
// The lane therefore needs every fourth element of a row.  Loading that
// directly (one dword per step, 16 rows per instruction) keeps the texture
// path busy for most of the kernel, so x is read in coalesced 16-byte pieces
// (a unit of 512/bs bf16 rows, one piece per lane) and transposed through
// the wave's own LDS: the piece of elements 8q .. 8q+7 is written as four
// dwords, dword r pairing elements 8q + r and 8q + 4 + r (one v_perm each),
// to row t, slot (r, q), so that lane (g, j) then reads its bs/4 elements as
// bs/8 consecutive dwords (one ds_read_b128 at bs 32).  Row strides of 20
// (bs 32) and 10 (bs 16) dwords make both sides bank-conflict-free.  T is
// staged the same way once per wave (row stride bs + 4 dwords) and its
// fragments kept in bs * bs / 64 VGPRs.  Four units of x are in flight ahead
// of the one computed.  fp32 x (weight packing) is read directly, one dword
// per step.
//
// The block maximum of token j is reduced over its four lane groups with two
// lane shuffles, each lane encodes its own outputs, and the code row of token
// j (16 bytes at bs 32, 8 at bs 16) is gathered into lane j with three more
// shuffles and stored once.
constexpr int kMfmaUnits = 8;     // units of x per wave
constexpr int kMfmaDepth = 4;     // units loaded ahead of the one computed

template <int BS, bool BF16>
struct XUnit {
  static constexpr int kRows = BF16 ? 512 / BS : 16;            // tokens per unit
  static constexpr int kGroups = kRows / 16;
  static constexpr int kRaw = BF16 ? 4 : BS / 4;                 // dwords per lane
  static constexpr int kStride = BF16 ? BS / 2 + BS / 8 : 0;     // LDS row stride of x in dwords (20, 10)
  static constexpr int kTStride = BS + 4;                        // LDS row stride of T
  static constexpr int kLdsDwords = BS * kTStride + kRows * kStride;
};

// Raw x of one unit starting at token tb (rows past n re-read row n - 1).
template <int BS, bool BF16>
__device__ __forceinline__ void load_unit(const void* X, int tb, int n, int d_in, size_t col, int lane,
                                          uint32_t (&raw)[XUnit<BS, BF16>::kRaw]) {
  if constexpr (BF16) {
    const int t = lane / (BS / 8), q = lane % (BS / 8);
    const uint16_t* p =
        reinterpret_cast<const uint16_t*>(X) + static_cast<size_t>(min(tb + t, n - 1)) * d_in + col + 8 * q;
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    raw[0] = v.x; raw[1] = v.y; raw[2] = v.z; raw[3] = v.w;
  } else {
    const int j = lane & 15, g = lane >> 4;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(X) + static_cast<size_t>(min(tb + j, n - 1)) * d_in + col + g;
#pragma unroll
    for (int c = 0; c < BS / 4; ++c) raw[c] = p[4 * c];
  }
}

// bf16 unit: raw pieces -> LDS rows in step order (see above)
template <int BS>
__device__ __forceinline__ void stage_unit(uint32_t* lx, int lane, const uint32_t (&raw)[4]) {
  constexpr int S = XUnit<BS, true>::kStride;
  const int t = lane / (BS / 8), q = lane % (BS / 8);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    lx[t * S + r * (BS / 8) + q] =
        __builtin_amdgcn_perm(raw[2 + (r >> 1)], raw[r >> 1], (r & 1) ? 0x07060302u : 0x05040100u);
}

// x values of group s of the unit for lane (g, j), in step order c = 0 .. bs/4 - 1
template <int BS, bool BF16>
__device__ __forceinline__ void group_x(const uint32_t* lx, const uint32_t (&raw)[XUnit<BS, BF16>::kRaw], int s,
                                        int lane, float (&xv)[BS / 4]) {
  if constexpr (BF16) {
    constexpr int S = XUnit<BS, true>::kStride;
    const int j = lane & 15, g = lane >> 4;
    const uint32_t* src = lx + (16 * s + j) * S + g * (BS / 8);
    uint32_t d[BS / 8];
    if constexpr (BS == 32) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(src);
      d[0] = v.x; d[1] = v.y;
    }
#pragma unroll
    for (int q = 0; q < BS / 8; ++q) {
      xv[2 * q] = __uint_as_float(d[q] << 16);
      xv[2 * q + 1] = __uint_as_float(d[q] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int c = 0; c < BS / 4; ++c) xv[c] = __uint_as_float(raw[c]);
  }
}

// Cross-row lane exchange without an LDS round trip: v_permlane16_swap of a
// value with itself yields, in every lane, the values of lanes l & ~16 and
// l | 16; v_permlane32_swap those of l & ~32 and l | 32 (checked on the GPU).
__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); }
__device__ __forceinline__ uint32_t max_xor16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t max_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t from_xor16(uint32_t v, bool odd_row) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return bitsel(0u - static_cast<uint32_t>(odd_row), r[0], r[1]);
}

// One 16-token group: the MFMA chains, then the block maximum, the encoders
// and the stores of token `tok` into row `row` (tok clamped to n - 1: a row
// past the end holds the inputs of row n - 1 and so writes its bytes again).
// Every lane stores, so the stores sit in straight-line code and the
// compiler's wait counts keep the loads ahead of them in flight (a store in a
// lane-masked branch makes every later wait assume it was not issued).
template <int BS, int FMT>
__device__ __forceinline__ void mfma_group(const float (&ta)[BS / 16][BS / 4], const float (&xv)[BS / 4], int gq,
                                           int row, int blk, int nblk, int d_in, float g,
                                           uint8_t* __restrict__ codes, void* __restrict__ scales,
                                           uint32_t& run_max) {
  constexpr int H = BS / 16, C = BS / 4;
  v4f acc[H];
#pragma unroll
  for (int h = 0; h < H; ++h) acc[h] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int h = 0; h < H; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[h][c], xv[c], acc[h], 0, 0, 0);
  float y[4 * H];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) y[4 * h + e] = acc[h][e];
  if constexpr (FMT == kApply) {
    float* dst = reinterpret_cast<float*>(codes) + static_cast<size_t>(row) * d_in + static_cast<size_t>(blk) * BS +
                 4 * gq;
#pragma unroll
    for (int h = 0; h < H; ++h)
      *reinterpret_cast<float4*>(dst + 16 * h) = make_float4(y[4 * h], y[4 * h + 1], y[4 * h + 2], y[4 * h + 3]);
    return;
  }
  uint32_t ab = 0;
#pragma unroll
  for (int k = 0; k < 4 * H; ++k) ab = max(ab, __float_as_uint(y[k]) & 0x7fffffffu);
  ab = max_xor32(max_xor16(ab));
  if constexpr (FMT == kAmax) {
    run_max = max(run_max, ab);                // rows past n repeat row n - 1
  } else {
    constexpr int QF = FMT == kMXP ? kMX : FMT;
    const BlockQuant<QF> q = block_quant<QF>(ab, g);
    uint32_t w[1];
    encode_pairs<QF, 2 * H>(y, q, w);
    // Lane group g holds code bytes 2g, 2g+1 (outputs 4g .. 4g+3) in its low
    // half and, at bs 32, bytes 8+2g, 9+2g in its high half.  Groups 2m and
    // 2m+1 together form dword m of the row (low halves) and, at bs 32,
    // dword 2 + m (high halves).  Group g stores dword g (bs 32) or g % 2
    // (bs 16, each dword twice); groups 1 and 2 take theirs from the other pair.
    // (selections as bit masks: written as conditionals they become branches)
    const uint32_t m_odd = 0u - static_cast<uint32_t>(gq & 1);
    const uint32_t p = from_xor16(w[0], gq & 1);
    const uint32_t ev = bitsel(m_odd, p, w[0]), od = bitsel(m_odd, w[0], p);   // the pair's even, odd lane words
    const uint32_t lo = (ev & 0xffffu) | (od << 16);
    uint32_t own = lo, send = lo;
    if constexpr (BS == 32) {
      const uint32_t hi = (ev >> 16) | (od & 0xffff0000u);
      own = bitsel(0u - static_cast<uint32_t>(gq == 3), hi, lo);
      send = bitsel(m_odd, lo, hi);
    }
    const auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
    const uint32_t other = bitsel(0u - static_cast<uint32_t>(gq < 2), r[1], r[0]);
    const uint32_t word = bitsel(0u - static_cast<uint32_t>(gq == 0 || gq == 3), own, other);
    uint8_t* dst = codes + static_cast<size_t>(row) * (d_in / 2) + static_cast<size_t>(blk) * (BS / 2);
    reinterpret_cast<uint32_t*>(dst)[BS == 32 ? gq : (gq & 1)] = word;
    if constexpr (FMT == kMXP)
      reinterpret_cast<uint8_t*>(scales)[mxfp4_plane_offset(row, blk, nblk / 8)] = static_cast<uint8_t>(q.scale);
    else
      store_scale<FMT>(scales, static_cast<size_t>(row) * nblk + blk, q.scale);
  }
}

template <int BS, int FMT, bool BF16>
// (X and T are not declared __restrict__ here: the compiler moves
// restrict-qualified loads freely and would issue x's before T's.)
__global__ __launch_bounds__(kWave * kWavesPerGroup) void tq_mfma_kernel(
    const void* X, const float* T, int n, int d_in, float g,
    uint8_t* __restrict__ codes, void* __restrict__ scales, uint32_t* __restrict__ amax_out,
    const int* __restrict__ tmap, int ngroups) {
  using U = XUnit<BS, BF16>;
  constexpr int H = BS / 16, C = BS / 4, D = kMfmaDepth;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kWavesPerGroup * U::kLdsDwords];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = d_in / BS;
  const int blk = blockIdx.x * kWavesPerGroup + wave;
  if (blk >= nblk) return;                       // wave-uniform; the waves share no LDS and meet at no barrier
  const int j = lane & 15, gq = lane >> 4;
  uint32_t* const lt = lds + wave * U::kLdsDwords;   // T, row stride kTStride
  uint32_t* const lx = lt + BS * U::kTStride;         // one unit of x
  // T's pieces are requested first, then the first units of x, so that the
  // wait for T (from L2) leaves the loads of x (from HBM) in flight
  const size_t col = static_cast<size_t>(blk) * BS;
  const int t0 = blockIdx.y * (kMfmaUnits * U::kRows);
  uint32_t run_max = 0;
  // the block's matrix, or with a group map its group's (ids clamped to the table)
  const int tsel = tmap ? min(max(tmap[blk], 0), ngroups - 1) : blk;
  const uint4* tp = reinterpret_cast<const uint4*>(T + static_cast<size_t>(tsel) * BS * BS);
  constexpr int NT = BS * BS / 256;   // pieces of T per lane (4 or 1)
  const uint4 tv0 = tp[lane];
  const uint4 tv1 = NT > 1 ? tp[lane + 64] : tv0;
  const uint4 tv2 = NT > 1 ? tp[lane + 128] : tv0;
  const uint4 tv3 = NT > 1 ? tp[lane + 192] : tv0;
  __builtin_amdgcn_sched_barrier(0);
  uint32_t raw[D][U::kRaw];
#pragma unroll
  for (int i = 0; i < D; ++i) load_unit<BS, BF16>(X, t0 + i * U::kRows, n, d_in, col, lane, raw[i]);
  __builtin_amdgcn_sched_barrier(0);
  // piece m = lane + 64 i of T: row m / (bs/4), columns 4 (m % (bs/4)) .. + 3
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int m = lane + 64 * i;
    *reinterpret_cast<uint4*>(lt + (m / (BS / 4)) * U::kTStride + 4 * (m % (BS / 4))) =
        i == 0 ? tv0 : i == 1 ? tv1 : i == 2 ? tv2 : tv3;
  }
  float ta[H][C];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int c = 0; c < C; ++c) ta[h][c] = __uint_as_float(lt[(16 * h + j) * U::kTStride + 4 * c + gq]);
  // Fully unrolled, so that every wait counts exactly the loads and stores
  // issued after the one it waits for.  Units past n repeat row n - 1, whose
  // bytes they write again unchanged.
#pragma unroll
  for (int u = 0; u < kMfmaUnits; ++u) {
    const int tb = t0 + u * U::kRows;
    if constexpr (BF16) stage_unit<BS>(lx, lane, raw[u % D]);
    float xv[U::kGroups][C];
#pragma unroll
    for (int s = 0; s < U::kGroups; ++s) group_x<BS, BF16>(lx, raw[u % D], s, lane, xv[s]);
    __builtin_amdgcn_sched_barrier(0);
    if (u + D < kMfmaUnits) load_unit<BS, BF16>(X, tb + D * U::kRows, n, d_in, col, lane, raw[u % D]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < U::kGroups; ++s)
      mfma_group<BS, FMT>(ta, xv[s], gq, min(tb + 16 * s + j, n - 1), blk, nblk, d_in, g, codes, scales, run_max);
  }
  if constexpr (FMT == kAmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
      run_max = max(run_max, static_cast<uint32_t>(__shfl_xor(static_cast<int>(run_max), off)));
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
    uint8_t* __restrict__ codes, void* __restrict__ scales, uint32_t* __restrict__ amax_out,
    const int* __restrict__ tmap, int ngroups) {
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

using KernelFn = void (*)(const void*, const float*, int, int, float, uint8_t*, void*, uint32_t*, const int*, int);

// bf16 x: the matrix-core kernel.  fp32 x still reads every fourth element
// with scattered dword loads there (no LDS transpose yet), which is slower
// than the vector-ALU kernel, so fp32 x keeps the latter.
template <int BS, int FMT>
KernelFn pick(bool bf16, bool ident) {
  if (bf16) return ident ? tq_kernel<BS, FMT, true, true> : tq_mfma_kernel<BS, FMT, true>;
  return ident ? tq_kernel<BS, FMT, false, true> : tq_kernel<BS, FMT, false, false>;
}

KernelFn select_kernel(int fmt, int bs, bool bf16, bool ident) {
  if (fmt == kMXP) return (bs == 32 && !ident) ? (bf16 ? tq_mfma_kernel<32, kMXP, true> : tq_mfma_kernel<32, kMXP, false>)
                                              : nullptr;
  if (fmt == kApply) {
    if (ident) return nullptr;
    if (bs == 32) return bf16 ? tq_mfma_kernel<32, kApply, true> : tq_mfma_kernel<32, kApply, false>;
    if (bs == 16) return bf16 ? tq_mfma_kernel<16, kApply, true> : tq_mfma_kernel<16, kApply, false>;
    return nullptr;
  }
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
                   uint8_t* codes, void* scales, uint32_t* amax, hipStream_t stream, const int* tmap = nullptr,
                   int ngroups = 0) {
  if (n == 0) return WUSH_OK;
  if (!wush::aligned16(T)) return wush::fail(WUSH_E_ARG, "transform_quant: T must be 16-byte aligned");
  KernelFn k = select_kernel(fmt, bs, bf16, T == nullptr);
  if (!k) return wush::fail(WUSH_E_UNSUPPORTED, "transform_quant: no kernel for fmt=%d bs=%d", fmt, bs);
  const int nblk = d_in / bs;
  const bool mfma = T && (bf16 || fmt == kApply || fmt == kMXP);
  const int per_wave = !mfma ? kTokensPerWave
                       : kMfmaUnits * (bs == 32 ? (bf16 ? XUnit<32, true>::kRows : XUnit<32, false>::kRows)
                                                : (bf16 ? XUnit<16, true>::kRows : XUnit<16, false>::kRows));
  dim3 grid((nblk + kWavesPerGroup - 1) / kWavesPerGroup, (n + per_wave - 1) / per_wave);
  if (grid.y > 65535u) return wush::fail(WUSH_E_SHAPE, "transform_quant: n=%d too large", n);
  hipLaunchKernelGGL(k, grid, dim3(kWave * kWavesPerGroup), 0, stream, X, T, n, d_in, g, codes, scales, amax, tmap,
                     ngroups);
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
  hipLaunchKernelGGL(k, grid, dim3(kWave * kWavesPerGroup), 0, stream, X, d, n, d_in, g, codes, scales, amax,
                     static_cast<const int*>(nullptr), 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "transform_quant_hd launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

// max|T x| over a tensor, written to a device uint (float bits).
// (T is a dense [nblk][bs][bs] matrix, or with hd the per-channel scales.)
wush_status tensor_amax(int bs, bool bf16, int n, int d_in, const void* X, const float* T, bool hd,
                        uint32_t* amax_dev, hipStream_t stream, const int* tmap, int ngroups) {
  hipLaunchKernelGGL(fill_u32, dim3(1), dim3(1), 0, stream, amax_dev, 0u);
  if (hd) return launch_hd(kAmax, bs, bf16, n, d_in, X, T, 0.0f, nullptr, nullptr, amax_dev, stream);
  return launch(kAmax, bs, bf16, n, d_in, X, T, 0.0f, nullptr, nullptr, amax_dev, stream, tmap, ngroups);
}

wush_status global_scale(int bs, bool bf16, int n, int d_in, const void* X, const float* T, bool hd, float* g_out,
                         hipStream_t stream, const int* tmap = nullptr, int ngroups = 0) {
  uint32_t* dbuf = nullptr;
  if (hipMalloc(&dbuf, sizeof(uint32_t)) != hipSuccess) return wush::fail(WUSH_E_HIP, "global_scale: hipMalloc failed");
  wush_status st = tensor_amax(bs, bf16, n, d_in, X, T, hd, dbuf, stream, tmap, ngroups);
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

size_t wush_mxfp4_planes_bytes(int rows, int K) {
  if (rows < 1 || K < 256 || K % 256 != 0) return 0;
  return static_cast<size_t>((rows + 255) / 256) * (K / 256) * 2048;
}

wush_status wush_transform_quant_mx_planes(wush_dtype xdt, int n, int d_in, const void* X, const float* Tx,
                                           uint8_t* codes, uint8_t* planes, void* stream) {
  wush_status st = check_common("wush_transform_quant_mx_planes", WUSH_MXFP4, n, d_in, X, codes, planes);
  if (st != WUSH_OK) return st;
  if (xdt != WUSH_F32 && xdt != WUSH_BF16) return wush::fail(WUSH_E_ARG, "wush_transform_quant_mx_planes: bad dtype");
  if (d_in % 256 != 0) return wush::fail(WUSH_E_SHAPE, "wush_transform_quant_mx_planes: d_in must be a multiple of 256");
  if (n > 0 && !Tx) return wush::fail(WUSH_E_ARG, "wush_transform_quant_mx_planes: needs a transform (Tx not NULL)");
  return launch(kMXP, 32, xdt == WUSH_BF16, n, d_in, X, Tx, 0.0f, codes, planes, nullptr,
                static_cast<hipStream_t>(stream));
}

wush_status wush_transform_apply(wush_dtype xdt, int bs, int n, int d_in, const void* X, const float* Tx, float* Y,
                                 void* stream) {
  if (bs != 16 && bs != 32) return wush::fail(WUSH_E_ARG, "wush_transform_apply: bs must be 16 or 32 (got %d)", bs);
  if (xdt != WUSH_F32 && xdt != WUSH_BF16) return wush::fail(WUSH_E_ARG, "wush_transform_apply: bad dtype");
  if (n < 0 || d_in < bs || d_in % bs != 0)
    return wush::fail(WUSH_E_SHAPE, "wush_transform_apply: need n >= 0 and d_in a positive multiple of %d", bs);
  if (n > 0 && (!X || !Tx || !Y)) return wush::fail(WUSH_E_ARG, "wush_transform_apply: null pointer");
  if (!wush::aligned16(X) || !wush::aligned16(Y))
    return wush::fail(WUSH_E_ARG, "wush_transform_apply: X and Y must be 16-byte aligned");
  return launch(kApply, bs, xdt == WUSH_BF16, n, d_in, X, Tx, 0.0f, reinterpret_cast<uint8_t*>(Y), nullptr, nullptr,
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

wush_status wush_transform_quant_shared(wush_format fmt, wush_dtype xdt, int n, int d_in, const void* X,
                                        const float* Tx, int ngroups, const int* group, float g, uint8_t* codes,
                                        void* scales, void* stream) {
  wush_status st = check_common("wush_transform_quant_shared", fmt, n, d_in, X, codes, scales);
  if (st != WUSH_OK) return st;
  if (xdt != WUSH_F32 && xdt != WUSH_BF16) return wush::fail(WUSH_E_ARG, "wush_transform_quant_shared: bad dtype");
  if (ngroups < 1) return wush::fail(WUSH_E_ARG, "wush_transform_quant_shared: ngroups must be >= 1");
  if (n > 0 && (!Tx || !group)) return wush::fail(WUSH_E_ARG, "wush_transform_quant_shared: null Tx or group map");
  if (fmt == WUSH_NVFP4 && !(g > 0.0f && g < 3.0e38f))
    return wush::fail(WUSH_E_ARG, "wush_transform_quant_shared: NVFP4 needs a positive finite tensor scale g");
  const int fk = fmt == WUSH_MXFP4 ? kMX : fmt == WUSH_NVFP4 ? kNV : kI4;
  return launch(fk, wush_format_block(fmt), xdt == WUSH_BF16, n, d_in, X, Tx, g, codes, scales, nullptr,
                static_cast<hipStream_t>(stream), group, ngroups);
}

wush_status wush_nvfp4_global_scale_shared(wush_dtype xdt, int n, int d_in, const void* X, const float* Tx,
                                           int ngroups, const int* group, float* g_out, void* stream) {
  if (!X || !Tx || !group || !g_out) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale_shared: null pointer");
  if (xdt != WUSH_F32 && xdt != WUSH_BF16)
    return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale_shared: bad dtype");
  if (ngroups < 1) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale_shared: ngroups must be >= 1");
  if (n < 1 || d_in < 16 || d_in % 16 != 0)
    return wush::fail(WUSH_E_SHAPE, "wush_nvfp4_global_scale_shared: need n >= 1 and d_in %% 16 == 0");
  if (!wush::aligned16(X)) return wush::fail(WUSH_E_ARG, "wush_nvfp4_global_scale_shared: X must be 16-byte aligned");
  return global_scale(16, xdt == WUSH_BF16, n, d_in, X, Tx, false, g_out, static_cast<hipStream_t>(stream), group,
                      ngroups);
}

wush_status wush_pack_weights_shared(wush_format fmt, int d_out, int d_in, const float* W, const float* Tw,
                                     int ngroups, const int* group, uint8_t* codes, void* scales, float* g_out,
                                     void* stream) {
  wush_status st = check_common("wush_pack_weights_shared", fmt, d_out, d_in, W, codes, scales);
  if (st != WUSH_OK) return st;
  if (ngroups < 1) return wush::fail(WUSH_E_ARG, "wush_pack_weights_shared: ngroups must be >= 1");
  if (d_out > 0 && (!Tw || !group)) return wush::fail(WUSH_E_ARG, "wush_pack_weights_shared: null Tw or group map");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float g = 0.0f;
  if (fmt == WUSH_NVFP4) {
    if (!g_out) return wush::fail(WUSH_E_ARG, "wush_pack_weights_shared: NVFP4 needs g_out");
    if (d_out < 1) return wush::fail(WUSH_E_SHAPE, "wush_pack_weights_shared: NVFP4 needs d_out >= 1");
    st = global_scale(16, false, d_out, d_in, W, Tw, false, &g, s, group, ngroups);
    if (st != WUSH_OK) return st;
    *g_out = g;
  } else if (g_out) {
    *g_out = 1.0f;
  }
  const int fk = fmt == WUSH_MXFP4 ? kMX : fmt == WUSH_NVFP4 ? kNV : kI4;
  return launch(fk, wush_format_block(fmt), false, d_out, d_in, W, Tw, g, codes, scales, nullptr, s, group, ngroups);
}

}  // extern "C"
