// Transform-then-quantize kernels for gfx950: the online activation step and
// the offline weight packing of WUSH.
//
// WUSH news article (chain.bitekongjian.com), deployment paragraph: at
// inference only the activations are transformed, one small matrix per block
// of input channels; weights are transformed and quantized once, offline.
// "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization" (AI Radio),
// "The gist": transform and quantizer run as one fused GPU kernel.
//
// Kernels:
//  * tq_dense_kernel: every non-identity block matrix, bf16 or fp32 x, all
//    formats, the unquantized values (wush_transform_apply) and the NVFP4
//    tensor maximum.  The transform runs on the fp32 matrix cores as a chain of
//    v_mfma_f32_16x16x4_f32, which reproduces the pinned FMA chain bit for bit;
//    each wave streams 16-token units of two adjacent 32-channel spans with the
//    next units' loads in flight (the workgroup's waves load whole lines
//    together and exchange them through LDS, from where each lane reads x in
//    the MFMA's step order), and encodes with the pinned block quantizers.
//  * tq_ident_kernel: the identity transform (a bit-exact copy), one block per
//    lane.
//  * tq_hd_kernel: the Hadamard-diagonal variant, one product and log2(bs)
//    butterfly stages per element on the vector ALU.
// The arithmetic is pinned (see wush.h): codes and scales are bit-exact
// functions of (T, x).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "common.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kTokensPerWave = 2 * kWave;   // identity kernel: two 64-token tiles per wave

// kApply: write y itself (fp32); kMXP: MXFP4 with the scales written in the
// plane order of the MXFP4 matmul's LDS stage (see mxfp4_plane_offset)
enum Fmt { kMX = 0, kNV = 1, kI4 = 2, kAmax = 3, kApply = 4, kMXP = 5 };

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Bit pattern of max |y[k]|: gfx950's v_maximum3_f32 with |.| source modifiers,
// three values per instruction.  It is the IEEE 754-2019 maximum, so a NaN
// anywhere propagates, and the result's bits order like the integer maximum of
// the |y| bit patterns: equal for finite and infinite values (subnormals kept,
// -0 and +0 both give 0), and at least 0x7f800001 when a NaN is present, which
// is all the block quantizers read from it.
template <int N>
__device__ __forceinline__ uint32_t abs_max_bits(const float* y) {
  float m = fabsf(y[0]);
#pragma unroll
  for (int k = 1; k < N; ++k) m = __builtin_elementwise_maximum(m, fabsf(y[k]));
  return __float_as_uint(m);
}

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

// Two E2M1 codes into byte `sel` of `old` (low nibble = a).  gfx950's packed FP4
// conversion rounds to nearest with ties to the even code, saturates at 6 and keeps
// the sign bit, which is exactly the pinned encoder for every non-NaN input.  Its
// scale operand s divides the values by the power of two that s's exponent field
// encodes, as an E8M0 byte (field 0 meaning 2^-127; checked on the GPU over zero,
// subnormal, tie and saturating blocks): s = 1.0 leaves them unchanged, and for
// MXFP4 s = the block scale 2^e replaces the multiplication by 2^-e.
__device__ __forceinline__ uint32_t cvt_pair_s(uint32_t old, float a, float b, float s, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 3);
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
  float div;        // MXFP4: the scale 2^e, applied by the conversion itself
  uint32_t scale;   // scale byte (E8M0, E4M3) or fp16 bits (INT4)
  bool zero;        // codes forced to 0
  bool soft;        // NVFP4 with 1/s not finite: the software encoder (0 * inf is NaN -> code 0)
};

template <int FMT>
__device__ __forceinline__ BlockQuant<FMT> block_quant(uint32_t ab, float g) {
  BlockQuant<FMT> q{1.0f, 1.0f, 0u, false, false};
  const bool bad = ab >= 0x7f800000u;          // NaN or Inf in the block
  if constexpr (FMT == kMX) {
    // 2^e = 2^(floor(log2 amax) - 2) as fp32 bits, the exponent field lowered by
    // 2 and clamped at 0 (one saturating subtract); its field is the E8M0 byte
    const uint32_t dbits = __builtin_elementwise_sub_sat(ab & 0x7f800000u, 0x01000000u);
    const uint32_t sbyte = dbits >> 23;                        // e + 127
    q.mul = __uint_as_float((254u - sbyte) << 23);             // 2^-e
    q.div = __uint_as_float(dbits);                            // 2^e, applied by the conversion
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
      for (int p = 0; p < NP; ++p) {
        if constexpr (FMT == kMX)
          w[p >> 2] = cvt_pair_s(w[p >> 2], y[2 * p], y[2 * p + 1], q.div, p & 3);
        else
          w[p >> 2] = cvt_pair_s(w[p >> 2], y[2 * p] * q.mul, y[2 * p + 1] * q.mul, 1.0f, p & 3);
      }
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
  const uint32_t ab = abs_max_bits<BS>(y);
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

// Identity transform (a bit-exact copy) with the three formats plus an
// amax-only pass (NVFP4 tensor scale).  A wave owns one block and two 64-token
// tiles: lane l quantizes tokens base + l and base + 64 + l, each block's
// values in one lane, so the block maximum needs no cross-lane reduction (an
// integer max of |y| bit patterns, which also flags NaN and Inf).
template <int BS, int FMT, bool BF16>
__global__ __launch_bounds__(kWave * kWavesPerGroup) __attribute__((amdgpu_waves_per_eu(4))) void tq_ident_kernel(
    const void* __restrict__ X, int n, int d_in, float g, uint8_t* __restrict__ codes, void* __restrict__ scales,
    uint32_t* __restrict__ amax_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = d_in / BS;
  const int blk = blockIdx.x * kWavesPerGroup + wave;
  if (blk >= nblk) return;                       // wave-uniform
  const int tok0 = blockIdx.y * (2 * kWave) + lane, tok1 = tok0 + kWave;
  uint32_t run_max = 0;
  float x0[BS], x1[BS];
  const size_t col = static_cast<size_t>(blk) * BS;
  if (tok0 < n) {
    load_block<BS, BF16>(X, static_cast<size_t>(tok0) * d_in + col, x0);
    encode_store<BS, FMT>(x0, static_cast<size_t>(tok0), blk, nblk, d_in, g, codes, scales, run_max);
  }
  if (tok1 < n) {
    load_block<BS, BF16>(X, static_cast<size_t>(tok1) * d_in + col, x1);
    encode_store<BS, FMT>(x1, static_cast<size_t>(tok1), blk, nblk, d_in, g, codes, scales, run_max);
  }
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
// flop per clock per SIMD, twice the vector FMA rate.  On this part vector-ALU
// instructions do not run under an fp32 MFMA (measured: their times add), so
// the kernel keeps its vector work per token small.
//
// Work unit: 16 tokens x one 32-channel span (one block at bs 32, two at
// bs 16).  A wave owns kSpans adjacent spans (128 bytes of every bf16 row,
// the four waves of a workgroup 512 contiguous bytes) and walks a run of
// units with the loads of the next kDepth units in flight.  Lane
// (g = l / 16, j = l % 16) works on token j of the unit.
//
// x: at step c the MFMA wants element 4c + g of the lane's token in lane
// group g, and the lane reads it from the workgroup's staging buffer (see the
// kernel).  bf16: elements 4c + g for c = 0 .. 7 are the low (g even) or high
// (g odd) halves of every other dword of the span, two in each 16-byte piece,
// so a lane reads them with one two-dword LDS read per piece and widens each
// with one v_perm (its two bytes on top, zeros below): no lane exchange.
// fp32: lane (q, j) reads elements 8q .. 8q+7 (32 bytes), and a 4 x 4
// transpose of dwords across the lane groups (two v_permlane32_swap and two
// v_permlane16_swap per four dwords) gives group g what it needs.
//
// T: at bs 32 the A operand row i of accumulator h is T row
// 8 (i / 4) + 4 h + i % 4.  Lane group g then ends with outputs 8g .. 8g+7 of
// its token (acc[0]: 8g .. 8g+3, acc[1]: 8g+4 .. 8g+7), whose four code
// bytes are contiguous: one dword store, no lane exchange.  At bs 16
// accumulator h is block h of the span, and lane group g holds outputs
// 4g .. 4g+3 of each block.  The fragments are loaded once per wave and
// transposed like fp32 x.
//
// Block maximum: over the lane's values, then over its token's four lane
// groups with two lane swaps; then the pinned block quantizers.
//
// Addressing: every load and store of a unit goes through a buffer resource
// whose base is the unit's first row (wave-uniform, in scalar registers) and
// whose size ends at the unit's last token inside [0, n); the lane's part is a
// 32-bit offset fixed for the whole run.  Tokens past n therefore read zeros
// and their stores are dropped by the resource's range check.  Plane-ordered
// scales interleave rows, so their stores carry a lane predicate instead.
// Spans (and at bs 16 blocks) past d_in repeat the last block, rewriting its
// bytes unchanged.  Every access stays inside the caller's buffers.
constexpr int kSpans = 2;    // 32-channel spans per wave
constexpr int kDepth = 4;    // units of x in flight ahead of the one computed

__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);   // a's lanes 32..63 <-> b's 0..31
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);   // a's odd rows <-> b's even rows
  a = r[0];
  b = r[1];
}
// 4 x 4 dword transpose across the lane groups (rows of 16 lanes): on entry
// d[r] of group q is D[q][r]; on exit d[q] of group r is D[q][r].
__device__ __forceinline__ void transpose4(uint32_t (&d)[4]) {
  swap32(d[0], d[2]);
  swap32(d[1], d[3]);
  swap16(d[0], d[1]);
  swap16(d[2], d[3]);
}

// maximum over the four lane groups of a token (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ uint32_t max_groups(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // values of lanes l & ~16, l | 16
  const uint32_t m = max(r[0], r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(m, m, false, false);   // values of lanes l & ~32, l | 32
  return max(t[0], t[1]);
}

// Maxima of two values over a token's four lane groups at once: on return
// every lane holds a's maximum in ma and b's in mb.  The first swap pairs rows
// (a0 b0 a2 b2 | a1 b1 a3 b3), the second folds rows 2-3 onto 0-1 (A B A B),
// the third spreads A and B over all four rows: three swaps and two maxima
// instead of four and four.
__device__ __forceinline__ void max_groups2(uint32_t a, uint32_t b, uint32_t& ma, uint32_t& mb) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  const uint32_t m = max(r[0], r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  const uint32_t mm = max(t[0], t[1]);
  const auto u = __builtin_amdgcn_permlane16_swap(mm, mm, false, false);
  ma = u[0];
  mb = u[1];
}

// First element of lane group q's eight in its token row, for span sp.
template <int BS>
__device__ __forceinline__ int span_col(int sp, int q, int nblk) {
  if constexpr (BS == 32) return min(sp, nblk - 1) * 32 + 8 * q;
  return min(2 * sp + (q >> 1), nblk - 1) * 16 + 8 * (q & 1);
}

template <bool BF16>
struct XRaw {
  static constexpr int kDwords = BF16 ? 4 : 8;
};

// Raw, unswizzled buffer resource of `bytes` bytes at `base` (dword 3 selects
// the 32-bit data format untyped accesses need on CDNA).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// One unit: its first token and how many of its 16 tokens lie inside [0, n)
// (0 past the end).  Both are wave-uniform.
struct Unit {
  size_t row0;
  uint32_t rows;
};
__device__ __forceinline__ Unit unit_at(int unit, int n) {
  // 32-bit unsigned arithmetic, so that it stays on the scalar unit
  const uint32_t r0 = static_cast<uint32_t>(unit) * 16u, nn = static_cast<uint32_t>(n);
  return Unit{static_cast<size_t>(r0), r0 >= nn ? 0u : min(nn - r0, 16u)};
}

// The unit's rows of an array of `row_bytes`-byte rows, as a buffer resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t unit_rsrc(const void* base, const Unit& un, uint32_t row_bytes) {
  return buf_rsrc(static_cast<const uint8_t*>(base) + un.row0 * row_bytes, un.rows * row_bytes);
}

// Stores through a unit's resource: lane offset v plus wave-uniform offset s.
__device__ __forceinline__ void st_b8(uint32_t x, __amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(x), r, v, s, 0);
}
__device__ __forceinline__ void st_b16(uint32_t x, __amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(x), r, v, s, 0);
}
__device__ __forceinline__ void st_b32(uint32_t x, __amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  __builtin_amdgcn_raw_buffer_store_b32(x, r, v, s, 0);
}
__device__ __forceinline__ void st_b64(uint32_t x, uint32_t y, __amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(v2u{x, y}, r, v, s, 0);
}
__device__ __forceinline__ void st_f4(float a, float b, float c, float d, __amdgpu_buffer_rsrc_t r, uint32_t v,
                                      uint32_t s) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(v4u{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c),
                                             __float_as_uint(d)},
                                         r, v, s, 0);
}

// Scale of (lane's token, block b) in the row-major scale array of a unit.
template <int FMT>
__device__ __forceinline__ void store_unit_scale(void* scales, const Unit& un, int nblk, int j, int b, uint32_t sc) {
  constexpr uint32_t ssz = FMT == kI4 ? 2u : 1u;
  const __amdgpu_buffer_rsrc_t r = unit_rsrc(scales, un, static_cast<uint32_t>(nblk) * ssz);
  if constexpr (FMT == kI4)
    st_b16(sc, r, static_cast<uint32_t>(j * nblk) * ssz, static_cast<uint32_t>(b) * ssz);
  else
    st_b8(sc, r, static_cast<uint32_t>(j * nblk), static_cast<uint32_t>(b));
}

// Plane-ordered scale of (lane's token, block 8 kb + bl), the layout of
// mxfp4_plane_offset: every row of a unit lies in one 256-row tile at one tile
// position, so the (tile, K block) region is a wave-uniform 2 KB base, and the
// lane adds plane bl's 256 bytes, 16 per token and the position rotated in odd
// planes.  kb must be wave-uniform.  Tokens past n (the last tile's planes hold
// rows past n) get an offset outside the 2 KB, which the range check drops.
__device__ __forceinline__ void store_plane_scale(void* scales, const Unit& un, int nblk, int j, int kb, int bl,
                                                  uint32_t sc) {
  const uint32_t r = static_cast<uint32_t>(un.row0) & 255u;
  const uint8_t* base = static_cast<const uint8_t*>(scales) + ((un.row0 >> 8) * static_cast<size_t>(nblk / 8) + kb) * 2048;
  const uint32_t pos0 = 8u * (r >> 7) + ((r >> 4) & 7u);
  const uint32_t off = static_cast<uint32_t>(bl) * 256u + 16u * static_cast<uint32_t>(j) + (pos0 ^ (8u * (bl & 1)));
  st_b8(sc, buf_rsrc(base, 2048u), static_cast<uint32_t>(j) < un.rows ? off : 0x80000000u, 0u);
}

// x operands of the eight MFMA steps of one span for lane (g, j), from the
// lane's 32 bytes of fp32 x (elements 8g .. 8g+7 of its token).
__device__ __forceinline__ void x_steps_f32(const uint32_t (&raw)[8], float (&xv)[8]) {
  uint32_t lo[4] = {raw[0], raw[1], raw[2], raw[3]}, hi[4] = {raw[4], raw[5], raw[6], raw[7]};
  transpose4(lo);
  transpose4(hi);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    xv[2 * q] = __uint_as_float(lo[q]);
    xv[2 * q + 1] = __uint_as_float(hi[q]);
  }
}

// A-operand fragments of one span: ta[h][c] = T[row][4c + g] for the rows
// described above (bs 32), or of block h of the span (bs 16, c < 4).  Loaded
// in raw form first (so that the loads of x can be issued before the wait for
// T), then transposed like fp32 x.
struct TRaw {
  uint4 v[4];
};

template <int BS>
__device__ __forceinline__ void load_t(const float* T, const int* tmap, int ngroups, int sp, int nblk, int q, int j,
                                       TRaw& tr) {
  if constexpr (BS == 32) {
    const int b = min(sp, nblk - 1);
    const int tsel = tmap ? min(max(tmap[b], 0), ngroups - 1) : b;
    const float* Tb = T + static_cast<size_t>(tsel) * 1024;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4* p = reinterpret_cast<const uint4*>(Tb + (8 * (j >> 2) + 4 * h + (j & 3)) * 32 + 8 * q);
      tr.v[2 * h] = p[0];
      tr.v[2 * h + 1] = p[1];
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = min(2 * sp + h, nblk - 1);
      const int tsel = tmap ? min(max(tmap[b], 0), ngroups - 1) : b;
      tr.v[h] = *reinterpret_cast<const uint4*>(T + static_cast<size_t>(tsel) * 256 + j * 16 + 4 * q);
    }
  }
}

template <int BS>
__device__ __forceinline__ void t_steps(const TRaw& tr, float (&ta)[2][8]) {
  if constexpr (BS == 32) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 a = tr.v[2 * h], c = tr.v[2 * h + 1];
      uint32_t lo[4] = {a.x, a.y, a.z, a.w}, hi[4] = {c.x, c.y, c.z, c.w};
      transpose4(lo);
      transpose4(hi);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ta[h][2 * k] = __uint_as_float(lo[k]);
        ta[h][2 * k + 1] = __uint_as_float(hi[k]);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t d[4] = {tr.v[h].x, tr.v[h].y, tr.v[h].z, tr.v[h].w};
      transpose4(d);
#pragma unroll
      for (int c = 0; c < 4; ++c) ta[h][c] = __uint_as_float(d[c]);
#pragma unroll
      for (int c = 4; c < 8; ++c) ta[h][c] = 0.0f;
    }
  }
}

// The MFMA chains, block maxima, encoders and stores of one span of one unit.
template <int BS, int FMT>
__device__ __forceinline__ void span_unit(const float (&ta)[2][8], const float (&xv)[8], int sp, int nblk, int q, int j,
                                          const Unit& un, int d_in, float g, uint8_t* __restrict__ codes,
                                          void* __restrict__ scales, uint32_t& run_max) {
  v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
  if constexpr (BS == 32) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[h][c], xv[c], acc[h], 0, 0, 0);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[h][c], xv[4 * h + c], acc[h], 0, 0, 0);
  }
  constexpr int QF = FMT == kMXP ? kMX : FMT;
  const uint32_t code_row = static_cast<uint32_t>(d_in / 2);
  if constexpr (BS == 32) {
    const int b = min(sp, nblk - 1);
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) { y[e] = acc[0][e]; y[4 + e] = acc[1][e]; }
    if constexpr (FMT == kApply) {
      const __amdgpu_buffer_rsrc_t r = unit_rsrc(codes, un, static_cast<uint32_t>(d_in) * 4u);
      const uint32_t v = static_cast<uint32_t>(j * d_in + 8 * q) * 4u, so = static_cast<uint32_t>(b) * 128u;
      st_f4(y[0], y[1], y[2], y[3], r, v, so);
      st_f4(y[4], y[5], y[6], y[7], r, v + 16u, so);
      return;
    }
    const uint32_t ab = max_groups(abs_max_bits<8>(y));
    if constexpr (FMT == kAmax) {
      run_max = max(run_max, ab);
    } else {
      const BlockQuant<QF> bq = block_quant<QF>(ab, g);
      uint32_t w[1];
      encode_pairs<QF, 4>(y, bq, w);
      st_b32(w[0], unit_rsrc(codes, un, code_row), static_cast<uint32_t>(j) * code_row + 4u * q,
             static_cast<uint32_t>(b) * 16u);
      if constexpr (FMT == kMXP)
        store_plane_scale(scales, un, nblk, j, b >> 3, b & 7, bq.scale);
      else
        store_unit_scale<QF>(scales, un, nblk, j, b, bq.scale);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = min(2 * sp + h, nblk - 1);
      float y[4] = {acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
      if constexpr (FMT == kApply) {
        st_f4(y[0], y[1], y[2], y[3], unit_rsrc(codes, un, static_cast<uint32_t>(d_in) * 4u),
              static_cast<uint32_t>(j * d_in + 4 * q) * 4u, static_cast<uint32_t>(b) * 64u);
        continue;
      }
      const uint32_t ab = max_groups(abs_max_bits<4>(y));
      if constexpr (FMT == kAmax) {
        run_max = max(run_max, ab);
      } else {
        const BlockQuant<QF> bq = block_quant<QF>(ab, g);
        uint32_t w[1];
        encode_pairs<QF, 2>(y, bq, w);
        st_b16(w[0], unit_rsrc(codes, un, code_row), static_cast<uint32_t>(j) * code_row + 2u * q,
               static_cast<uint32_t>(b) * 8u);
        store_unit_scale<QF>(scales, un, nblk, j, b, bq.scale);
      }
    }
  }
}

// Both spans of a unit at bs 32 (blocks b0 and b0 + 1, both inside d_in),
// quantized, with their stores merged: the two code dwords of lane group g
// (bytes 4g.. of block b0 and of block b0 + 1) are exchanged across the lane
// groups so that group g holds bytes 8g .. 8g+7 of the token's 32-byte run,
// one 8-byte store; the two scales go out in one store, lane groups 0 and 2
// writing block b0's and groups 1 and 3 block b0 + 1's.
template <int FMT>
__device__ __forceinline__ void pair_unit(const float (&ta)[2][2][8], const float (&xv)[2][8], int b0, int nblk, int q,
                                          int j, const Unit& un, int d_in, float g, uint8_t* __restrict__ codes,
                                          void* __restrict__ scales) {
  constexpr int QF = FMT == kMXP ? kMX : FMT;
  float y[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[s][h][c], xv[s][c], acc[h], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) { y[s][e] = acc[0][e]; y[s][4 + e] = acc[1][e]; }
  }
  uint32_t ab[2];
  max_groups2(abs_max_bits<8>(y[0]), abs_max_bits<8>(y[1]), ab[0], ab[1]);
  uint32_t w[2], sc[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const BlockQuant<QF> bq = block_quant<QF>(ab[s], g);
    uint32_t ws[1];
    encode_pairs<QF, 4>(y[s], bq, ws);
    w[s] = ws[0];
    sc[s] = bq.scale;
  }
  swap32(w[0], w[1]);
  swap16(w[0], w[1]);
  const uint32_t code_row = static_cast<uint32_t>(d_in / 2);
  st_b64(w[0], w[1], unit_rsrc(codes, un, code_row), static_cast<uint32_t>(j) * code_row + 8u * q,
         static_cast<uint32_t>(b0) * 16u);
  const int odd = q & 1;
  const uint32_t scale = odd ? sc[1] : sc[0];
  if constexpr (FMT == kMXP)   // b0 is even: both blocks share their 256-wide K block
    store_plane_scale(scales, un, nblk, j, b0 >> 3, (b0 & 7) + odd, scale);
  else
    store_unit_scale<QF>(scales, un, nblk, j, b0 + odd, scale);
}

// Every lane receives the value v of each of its token's four lane groups:
// o[r] = v of lane group r (three lane swaps).
__device__ __forceinline__ void gather_groups(uint32_t v, uint32_t (&o)[4]) {
  const auto t = __builtin_amdgcn_permlane16_swap(v, v, false, false);     // rows: (v0 v0 v2 v2), (v1 v1 v3 v3)
  const auto u = __builtin_amdgcn_permlane32_swap(t[0], t[0], false, false);
  const auto w = __builtin_amdgcn_permlane32_swap(t[1], t[1], false, false);
  o[0] = u[0];
  o[1] = w[0];
  o[2] = u[1];
  o[3] = w[1];
}

// NVFP4 (bs 16): the four blocks of a unit's two spans (blocks 2 sp0 .. 2 sp0
// + 3, all inside d_in), with the scale work split over the lane groups.  A
// block's scale takes two correctly rounded divisions and the E4M3 rounding,
// about forty vector instructions; every lane of a token would compute the
// same four.  Instead the block maxima are reduced so that lane group r ends
// with block r's (two swaps per pair of blocks, one more between the pairs),
// each lane computes that one block's multiplier, scale and flags, and the
// lanes gather the four multipliers and flags back (three swaps each).  The
// 2-byte code pieces (lane group r holds bytes 2r, 2r+1 of every block) are
// then transposed so that lane group r holds block r's 8 bytes: one 8-byte
// code store and one scale store per lane.
template <int FMT>
__device__ __forceinline__ void quad_unit(const float (&ta)[2][2][8], const float (&xv)[2][8], int sp0, int nblk, int q,
                                          int j, const Unit& un, int d_in, float g, uint8_t* __restrict__ codes,
                                          void* __restrict__ scales) {
  static_assert(FMT == kNV, "quad path: NVFP4");
  float y[4][4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[s][h][c], xv[s][4 * h + c], acc[h], 0, 0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[2 * s + h][e] = acc[h][e];
  }
  // maxima: after the pair swaps row r holds blocks (0, 1) or (2, 3) over two
  // rows each; the swap between the row pairs folds them to block r in row r
  const auto r01 = __builtin_amdgcn_permlane16_swap(abs_max_bits<4>(y[0]), abs_max_bits<4>(y[1]), false, false);
  const auto r23 = __builtin_amdgcn_permlane16_swap(abs_max_bits<4>(y[2]), abs_max_bits<4>(y[3]), false, false);
  const auto f = __builtin_amdgcn_permlane32_swap(max(r01[0], r01[1]), max(r23[0], r23[1]), false, false);
  const BlockQuant<kNV> own = block_quant<kNV>(max(f[0], f[1]), g);
  uint32_t mul[4], flg[4];
  gather_groups(__float_as_uint(own.mul), mul);
  gather_groups(own.scale | (own.zero ? 0x100u : 0u) | (own.soft ? 0x200u : 0u), flg);
  uint32_t c16[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const BlockQuant<kNV> bq{__uint_as_float(mul[b]), 1.0f, flg[b] & 0xffu, (flg[b] & 0x100u) != 0u,
                             (flg[b] & 0x200u) != 0u};
    uint32_t w[1];
    encode_pairs<kNV, 2>(y[b], bq, w);
    c16[b] = w[0];
  }
  // 4 x 4 transpose of 2-byte pieces across the lane groups
  uint32_t p0 = (c16[0] & 0xffffu) | (c16[1] << 16), p1 = (c16[2] & 0xffffu) | (c16[3] << 16);
  swap32(p0, p1);                                           // rows 0-1: blocks 0, 1; rows 2-3: blocks 2, 3
  uint32_t q0 = __builtin_amdgcn_perm(p1, p0, 0x05040100u); // low pieces of p0, p1
  uint32_t q1 = __builtin_amdgcn_perm(p1, p0, 0x07060302u); // high pieces
  swap16(q0, q1);
  const uint32_t d0 = __builtin_amdgcn_perm(q1, q0, 0x05040100u);
  const uint32_t d1 = __builtin_amdgcn_perm(q1, q0, 0x07060302u);
  const uint32_t code_row = static_cast<uint32_t>(d_in / 2);
  st_b64(d0, d1, unit_rsrc(codes, un, code_row), static_cast<uint32_t>(j) * code_row + 8u * q,
         static_cast<uint32_t>(2 * sp0) * 8u);
  store_unit_scale<kNV>(scales, un, nblk, j, 2 * sp0 + q, own.scale);
}

// Does the merged-store path apply?  bs 32 with an even number of blocks (two
// blocks per wave, a pair of 2-byte scales aligned), or NVFP4 at bs 16 with a
// multiple of four blocks (four per wave), so that every wave's blocks lie
// inside d_in.
constexpr bool pair_format(int bs, int fmt) {
  return (bs == 32 && (fmt == kMX || fmt == kI4 || fmt == kMXP)) || (bs == 16 && fmt == kNV);
}

// Vector-memory stores one unit issues (for the prologue above).
template <int BS, int FMT, bool PAIR>
constexpr int stores_per_unit() {
  if constexpr (FMT == kAmax) return 0;
  else if constexpr (PAIR) return 2;                        // codes of both blocks, one scale
  else if constexpr (FMT == kApply) return kSpans * 2;      // two float4 per span (bs 16: one per block)
  else if constexpr (BS == 32) return kSpans * 2;           // codes and scale per span
  else return kSpans * 4;                                   // codes and scale per block, two blocks per span
}
constexpr bool kMatchEntry = true;

// One unit of all the wave's spans: merged stores (PAIR), else span by span.
template <int BS, int FMT, bool PAIR>
__device__ __forceinline__ void unit_out(const float (&ta)[kSpans][2][8], const float (&xv)[kSpans][8], int sp0,
                                         int nblk, int q, int j, const Unit& un, int d_in, float g,
                                         uint8_t* __restrict__ codes, void* __restrict__ scales, uint32_t& run_max) {
  if constexpr (PAIR) {
    static_assert(kSpans == 2 && pair_format(BS, FMT), "merged stores: two spans of a quantized format");
    if constexpr (BS == 32)
      pair_unit<FMT>(ta, xv, sp0, nblk, q, j, un, d_in, g, codes, scales);
    else
      quad_unit<FMT>(ta, xv, sp0, nblk, q, j, un, d_in, g, codes, scales);
  } else {
#pragma unroll
    for (int s = 0; s < kSpans; ++s)
      span_unit<BS, FMT>(ta[s], xv[s], sp0 + s, nblk, q, j, un, d_in, g, codes, scales, run_max);
  }
}

// Workgroup barrier for the x staging buffers: this wave's LDS traffic done,
// then s_barrier.  No wait on the vector-memory counter, so the loads of the
// units ahead stay in flight across it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte piece of x for the staging buffer: offset v within the unit's rows.
template <bool STREAM>
__device__ __forceinline__ uint4 load_piece(const void* X, const Unit& un, uint32_t row_bytes, uint32_t v) {
  constexpr int kPolicy = STREAM ? 2 : 0;
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(unit_rsrc(X, un, row_bytes), v, 0, kPolicy));
}

// (X and T are not declared __restrict__: restrict-qualified loads would be
// moved freely across the scheduling fences.)
//
// x loads: the four waves of a workgroup cover 16 tokens x 512 contiguous
// bytes of x per unit (fp32: 1 KB), so each load instruction reads whole
// 128-byte lines of two rows (fp32: one row), 512 bytes of each; a wave puts
// its pieces into an LDS staging buffer (two buffers, one per unit parity,
// 16-byte chunks XOR-swizzled by row & 15, so that the 16 tokens of a read
// fall in 16 different chunks) and, after one workgroup barrier per unit,
// reads what its lanes compute on: bf16 lane (g, j) the dwords of token j
// holding elements 4c + g, fp32 lane (q, j) the 32 bytes of token j at
// span_col.  A wave whose
// spans all lie past d_in still loads and stages its share and meets every
// barrier; its stores go to a unit of no rows.
template <int BS, int FMT, bool BF16, bool PAIR, bool STREAM>
__global__ __launch_bounds__(kWave * kWavesPerGroup) void tq_dense_kernel(
    const void* X, const float* T, int n, int d_in, float g, uint8_t* __restrict__ codes, void* __restrict__ scales,
    uint32_t* __restrict__ amax_out, const int* __restrict__ tmap, int ngroups, int upw) {
  constexpr int R = XRaw<BF16>::kDwords;
  constexpr uint32_t kEsz = BF16 ? 2u : 4u;
  constexpr int kLd = R / 2;                                     // 1 KB load instructions per wave and unit
  constexpr int kRowBytes = kWavesPerGroup * kSpans * 32 * kEsz; // the workgroup's bytes of one row
  constexpr int kRowsPerLd = 1024 / kRowBytes;
  constexpr int kLanesPerRow = kWave / kRowsPerLd;
  __shared__ __attribute__((aligned(16))) uint8_t xstage[2][16 * kRowBytes];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, q = lane >> 4;
  const int nblk = d_in / BS;
  const int nspans = (d_in + 31) / 32;
  const int sp0 = (blockIdx.x * kWavesPerGroup + wave) * kSpans;
  const bool active = sp0 < nspans;               // wave-uniform
  const int u0 = blockIdx.y * upw;                // first unit (16 tokens) of this workgroup
  const uint32_t row_bytes = static_cast<uint32_t>(d_in) * kEsz;
  // the lane's loads (offset within the unit's rows) and their staging slots
  uint32_t xoff[kLd], soff[kLd];
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int row = (wave * kLd + i) * kRowsPerLd + lane / kLanesPerRow, ch = lane % kLanesPerRow;
    xoff[i] = static_cast<uint32_t>(row) * row_bytes + blockIdx.x * static_cast<uint32_t>(kRowBytes) + ch * 16u;
    soff[i] = static_cast<uint32_t>(row * kRowBytes + ((ch ^ (row & 15)) * 16));
  }
  // the lane's reads: token j's pieces at span_col of each span (a clamped
  // span reads the last block, which lies in this workgroup's segment)
  constexpr int kReads = BF16 ? 4 : R / 4;
  uint32_t roff[kSpans][kReads];
#pragma unroll
  for (int s = 0; s < kSpans; ++s) {
    if constexpr (BF16) {
      // bf16: lane group q takes elements 4c + q of its token (c = 0 .. 7),
      // the low (q even) or high (q odd) half of every other dword: two per
      // 16-byte piece h, which holds elements 8h .. 8h + 7 of the span
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int col = active ? span_col<BS>(sp0 + s, h, nblk) - static_cast<int>(blockIdx.x) * (kRowBytes / 2) : 0;
        roff[s][h] = static_cast<uint32_t>(j * kRowBytes + (((col / 8) ^ (j & 15)) * 16) + (q >> 1) * 4);
      }
    } else {
      const int col = active ? span_col<BS>(sp0 + s, q, nblk) - static_cast<int>(blockIdx.x) * (kRowBytes / static_cast<int>(kEsz)) : 0;
#pragma unroll
      for (int h = 0; h < R / 4; ++h) {
        const int ch = col * static_cast<int>(kEsz) / 16 + h;
        roff[s][h] = static_cast<uint32_t>(j * kRowBytes + ((ch ^ (j & 15)) * 16));
      }
    }
  }
  // bf16 -> fp32 of the half a lane group takes: its two bytes on top, zeros below
  const uint32_t xsel = (q & 1) ? 0x03020c0cu : 0x01000c0cu;
  // T's loads first, then the first units of x; the wait for T (from L2)
  // then leaves the loads of x (from HBM) in flight
  TRaw traw[kSpans];
#pragma unroll
  for (int s = 0; s < kSpans; ++s) load_t<BS>(T, tmap, ngroups, sp0 + s, nblk, q, j, traw[s]);
  __builtin_amdgcn_sched_barrier(0);
  uint4 ld[kDepth][kLd];
  // Loads and stores retire through one in-order counter, and the loop's
  // waits are shared by all its iterations: each unit's loads are followed by
  // the previous unit's stores in the loop, so here each unit's loads are
  // followed by as many stores that write nothing (a resource of size 0).
  // The compiler then sees the same count of later operations before every
  // wait for a unit's loads, on entry and in steady state, and waits for that
  // unit's loads only, not for the units after it and the stores between.
  const __amdgpu_buffer_rsrc_t nowhere = buf_rsrc(codes, 0u);
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    const Unit un = unit_at(u0 + d, n);
#pragma unroll
    for (int i = 0; i < kLd; ++i) ld[d][i] = load_piece<STREAM>(X, un, row_bytes, xoff[i]);
    if constexpr (kMatchEntry) {
#pragma unroll
      for (int k = 0; k < stores_per_unit<BS, FMT, PAIR>(); ++k) st_b32(0u, nowhere, 256u * (kDepth * d + k), 0u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float ta[kSpans][2][8];
#pragma unroll
  for (int s = 0; s < kSpans; ++s) t_steps<BS>(traw[s], ta[s]);
  uint32_t run_max = 0;
  // unit d's pieces through staging buffer d % 2 into the lane's x operands
  auto exchange = [&](int d, float (&xv)[kSpans][8]) {
    uint8_t* const st = xstage[d & 1];
#pragma unroll
    for (int i = 0; i < kLd; ++i) *reinterpret_cast<uint4*>(st + soff[i]) = ld[d][i];
    stage_barrier();
#pragma unroll
    for (int s = 0; s < kSpans; ++s) {
      if constexpr (BF16) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t* p = reinterpret_cast<const uint32_t*>(st + roff[s][h]);
          xv[s][2 * h] = __uint_as_float(__builtin_amdgcn_perm(p[0], p[0], xsel));
          xv[s][2 * h + 1] = __uint_as_float(__builtin_amdgcn_perm(p[2], p[2], xsel));
        }
      } else {
        uint32_t xr[R];
#pragma unroll
        for (int h = 0; h < R / 4; ++h) {
          const uint4 v = *reinterpret_cast<const uint4*>(st + roff[s][h]);
          xr[4 * h] = v.x; xr[4 * h + 1] = v.y; xr[4 * h + 2] = v.z; xr[4 * h + 3] = v.w;
        }
        x_steps_f32(xr, xv[s]);
      }
    }
  };
  // the unit a wave stores to: its own, or none for a wave past d_in
  auto out_unit = [&](int unit) { return active ? unit_at(unit, n) : Unit{0, 0u}; };
  // Units u0 .. u0 + upw - 1 (upw a multiple of kDepth), the last kDepth of
  // them without refills.
  int u = 0;
#pragma unroll 1
  for (; u + kDepth < upw; u += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      float xv[kSpans][8];
      exchange(d, xv);
      __builtin_amdgcn_sched_barrier(0);
      const Unit nx = unit_at(u0 + u + d + kDepth, n);
#pragma unroll
      for (int i = 0; i < kLd; ++i) ld[d][i] = load_piece<STREAM>(X, nx, row_bytes, xoff[i]);
      __builtin_amdgcn_sched_barrier(0);
      unit_out<BS, FMT, PAIR>(ta, xv, sp0, nblk, q, j, out_unit(u0 + u + d), d_in, g, codes, scales, run_max);
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    float xv[kSpans][8];
    exchange(d, xv);
    unit_out<BS, FMT, PAIR>(ta, xv, sp0, nblk, q, j, out_unit(u0 + u + d), d_in, g, codes, scales, run_max);
  }
  if constexpr (FMT == kAmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
      run_max = max(run_max, static_cast<uint32_t>(__shfl_xor(static_cast<int>(run_max), off)));
    if (lane == 0 && active) atomicMax(amax_out, run_max);
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
using DenseFn = void (*)(const void*, const float*, int, int, float, uint8_t*, void*, uint32_t*, const int*, int, int);
using IdentFn = void (*)(const void*, int, int, float, uint8_t*, void*, uint32_t*);

// Merged-store kernels stream x with non-temporal loads when x is larger than
// the 256 MB Infinity Cache, which then cannot keep it for a later kernel
// anyway (Qwen3-14B down projection, 570 MB of bf16 x: 218-220 against
// 235-237 us); on smaller x the default policy is as fast or slightly faster.
constexpr size_t kStreamBytes = size_t{256} << 20;

template <int BS, int FMT>
DenseFn dense(bool bf16, bool pair, bool stream) {
  if constexpr (pair_format(BS, FMT)) {
    if (pair && stream)
      return bf16 ? tq_dense_kernel<BS, FMT, true, true, true> : tq_dense_kernel<BS, FMT, false, true, true>;
    if (pair) return bf16 ? tq_dense_kernel<BS, FMT, true, true, false> : tq_dense_kernel<BS, FMT, false, true, false>;
  }
  return bf16 ? tq_dense_kernel<BS, FMT, true, false, false> : tq_dense_kernel<BS, FMT, false, false, false>;
}

DenseFn select_dense(int fmt, int bs, bool bf16, int nblk, bool stream) {
  const bool pair = bs == 32 ? nblk % 2 == 0 : nblk % 4 == 0;
  if (bs == 32) {
    switch (fmt) {
      case kMX: return dense<32, kMX>(bf16, pair, stream);
      case kI4: return dense<32, kI4>(bf16, pair, stream);
      case kAmax: return dense<32, kAmax>(bf16, pair, stream);
      case kApply: return dense<32, kApply>(bf16, pair, stream);
      case kMXP: return dense<32, kMXP>(bf16, pair, stream);
    }
  } else if (bs == 16) {
    switch (fmt) {
      case kNV: return dense<16, kNV>(bf16, pair, stream);
      case kAmax: return dense<16, kAmax>(bf16, pair, stream);
      case kApply: return dense<16, kApply>(bf16, pair, stream);
    }
  }
  return nullptr;
}

template <int BS, int FMT>
IdentFn ident(bool bf16) { return bf16 ? tq_ident_kernel<BS, FMT, true> : tq_ident_kernel<BS, FMT, false>; }

IdentFn select_ident(int fmt, int bs, bool bf16) {
  if (bs == 32) {
    switch (fmt) {
      case kMX: return ident<32, kMX>(bf16);
      case kI4: return ident<32, kI4>(bf16);
      case kAmax: return ident<32, kAmax>(bf16);
    }
  } else if (bs == 16) {
    switch (fmt) {
      case kNV: return ident<16, kNV>(bf16);
      case kAmax: return ident<16, kAmax>(bf16);
    }
  }
  return nullptr;
}

// Units (16 tokens) per wave of the dense kernel: about sixteen waves per
// SIMD over the whole grid (four resident at a time, so several rounds, and
// short runs that keep the last round's imbalance small), at least kDepth
// units each, a multiple of kDepth.
int dense_units_per_wave(int n, int d_in) {
  const long units = (n + 15) / 16;
  const long span_groups = ((d_in + 31) / 32 + kSpans - 1) / kSpans;
  const long wave_cols = (span_groups + kWavesPerGroup - 1) / kWavesPerGroup * kWavesPerGroup;
  const long target_waves = 16L * 4 * 256;    // 16 waves on each of the 1024 SIMDs
  const long slices = std::max(1L, target_waves / wave_cols);
  long upw = (units + slices - 1) / slices;
  upw = (upw + kDepth - 1) / kDepth * kDepth;
  upw = std::max<long>(upw, kDepth);
  while ((units + upw - 1) / upw > 65535) upw += kDepth;
  return static_cast<int>(upw);
}

wush_status launch(int fmt, int bs, bool bf16, int n, int d_in, const void* X, const float* T, float g,
                   uint8_t* codes, void* scales, uint32_t* amax, hipStream_t stream, const int* tmap = nullptr,
                   int ngroups = 0) {
  if (n == 0) return WUSH_OK;
  if (!wush::aligned16(T)) return wush::fail(WUSH_E_ARG, "transform_quant: T must be 16-byte aligned");
  if (!T) {
    IdentFn k = select_ident(fmt, bs, bf16);
    if (!k) return wush::fail(WUSH_E_UNSUPPORTED, "transform_quant: no identity kernel for fmt=%d bs=%d", fmt, bs);
    const int nblk = d_in / bs;
    dim3 grid((nblk + kWavesPerGroup - 1) / kWavesPerGroup, (n + kTokensPerWave - 1) / kTokensPerWave);
    if (grid.y > 65535u) return wush::fail(WUSH_E_SHAPE, "transform_quant: n=%d too large", n);
    hipLaunchKernelGGL(k, grid, dim3(kWave * kWavesPerGroup), 0, stream, X, n, d_in, g, codes, scales, amax);
  } else {
    const bool streamed = static_cast<size_t>(n) * static_cast<size_t>(d_in) * (bf16 ? 2u : 4u) > kStreamBytes;
    DenseFn k = select_dense(fmt, bs, bf16, d_in / bs, streamed);
    if (!k) return wush::fail(WUSH_E_UNSUPPORTED, "transform_quant: no kernel for fmt=%d bs=%d", fmt, bs);
    const int upw = dense_units_per_wave(n, d_in);
    const int span_groups = ((d_in + 31) / 32 + kSpans - 1) / kSpans;
    dim3 grid((span_groups + kWavesPerGroup - 1) / kWavesPerGroup, ((n + 15) / 16 + upw - 1) / upw);
    hipLaunchKernelGGL(k, grid, dim3(kWave * kWavesPerGroup), 0, stream, X, T, n, d_in, g, codes, scales, amax, tmap,
                       ngroups, upw);
  }
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
