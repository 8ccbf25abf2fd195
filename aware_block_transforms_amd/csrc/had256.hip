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
// vector maximum, an fp16 scale and codes q in [-3, 3].  The codes are stored
// as c = q + 4 in records of 16 rows x 256 codes laid out for the GEMV's
// loads: per (16-row block, chunk) 1568 bytes = 64 lanes x 16 bytes of code
// bits 0-1, 64 lanes x 8 bytes of code bit 2, and the 16 fp16 scales.  Lane
// l = 16 g + r holds row r's codes 64 g .. 64 g + 63; byte m of its 16 holds
// codes 64 g + 16 t + m (t = 0..3) at bits 2 t, and byte 4 j + b of its 8
// holds bit 2 of code 64 g + 16 (u / 2) + 8 j + 4 (u % 2) + b at bit u.
//
// GEMV: instead of inverse-rotating every weight (8 butterflies per weight on
// the vector ALU), the rotation is moved to the activations, which every
// output row shares:  sum_k x_k * (s/16)(H q)_k = (s/16) * sum_m q_m (H x)_m
// because H is symmetric.  The activations of each chunk are rotated once and
// split into two int8 terms; the weight stream then only unpacks codes to
// int8 (a shift and a masked merge per 4 codes) and the dot products run on
// the int8 matrix cores.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

constexpr int kVec = 256;
constexpr int kBlockRows = 16;
constexpr int kRecord = 1568;      // per (16-row block, chunk)
constexpr int kHiPlane = 1024;     // offset of the bit-2 plane in a record
constexpr int kScales = 1536;      // offset of the 16 fp16 scales

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

// One workgroup per (row, chunk) over the rows padded to a multiple of 16;
// padding rows are zero vectors (codes q = 0, scale 0).
__global__ __launch_bounds__(kVec) void had256_pack_kernel(const float* __restrict__ W, int d_out, int d_in,
                                                           uint8_t* __restrict__ packed) {
  __shared__ float v[kVec];
  __shared__ uint32_t wmax[kVec / 64];
  __shared__ uint8_t cc[kVec];
  const int t = threadIdx.x;
  const int nv = d_in / kVec;
  const size_t vec = blockIdx.x;                 // row * nv + chunk
  const int row = static_cast<int>(vec / nv), c = static_cast<int>(vec % nv);
  const float x = (row < d_out) ? W[static_cast<size_t>(row) * d_in + c * kVec + t] : 0.0f;
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
  cc[t] = static_cast<uint8_t>(q + 4);
  __syncthreads();
  const int r = row % kBlockRows;
  uint8_t* rec = packed + (static_cast<size_t>(row / kBlockRows) * nv + c) * kRecord;
  if (t < 64) {
    // bits 0-1: lane 16 g + r, byte m
    const int g = t >> 4, m = t & 15;
    uint32_t byte = 0;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) byte |= (cc[64 * g + 16 * tt + m] & 3u) << (2 * tt);
    rec[16 * (16 * g + r) + m] = static_cast<uint8_t>(byte);
  } else if (t < 96) {
    // bit 2: lane 16 g + r, byte 4 j + b
    const int i = t - 64, g = i >> 3, hb = i & 7, j = hb >> 2, b = hb & 3;
    uint32_t byte = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) byte |= ((cc[64 * g + 16 * (u >> 1) + 8 * j + 4 * (u & 1) + b] >> 2) & 1u) << u;
    rec[kHiPlane + 8 * (16 * g + r) + hb] = static_cast<uint8_t>(byte);
  }
  if (t == 0) {
    uint16_t hb;
    __builtin_memcpy(&hb, &h, 2);
    *reinterpret_cast<uint16_t*>(rec + kScales + 2 * r) = hb;
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

// ---------------------------------------------------------------------------
// GEMV on the int8 matrix cores.
//
// Per 256-chunk c and batch row b the rotated activations v = H x_c (fp32,
// unnormalised butterflies) are split as v ~ sigma (a_hi + a_lo / 128) with
// sigma = max|v| / 127 and int8 a_hi = rint(v / sigma), a_lo = rint((v /
// sigma - a_hi) * 128); the dropped part is below sigma / 256 per element.
// Then per weight row and chunk
//   sum_m q_m v_m ~ sigma * (sum_m q_m a_hi_m + (sum_m q_m a_lo_m) / 128)
// with both sums exact in int32 (v_mfma_i32_16x16x64_i8 on the stored codes
// c = q + 4, the accumulators starting at -4 sum_m a_m), and
//   y[b][row] = sum_c (s / 16) * that, accumulated in fp32.
//
// K order: MFMA t of lane group g takes codes 64 g + 16 t .. + 15 in natural
// order, so the activation operand of a chunk is its int8 vector as stored.

constexpr int kGemvWaves = 16;     // K split inside a workgroup: wave w takes chunks w, w + 16, ...
constexpr int kGemvTiles = 4;      // 16-row MFMA tiles (row blocks) per workgroup
constexpr int kGemvRows = kBlockRows * kGemvTiles;
constexpr int kFusedBatch = 4;     // batches up to this size rotate their activations inside the GEMV

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Orders this wave's LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Entry (a, b) of the 16-point Sylvester Hadamard matrix, (-1)^popcount(a & b).
__device__ __forceinline__ float hsign(int a, int b) { return (__builtin_popcount(a & b) & 1) ? -1.0f : 1.0f; }

// Wave-wide max / sum: DPP butterflies inside each 16-lane row (xor 1, xor 2,
// then the half-row and row mirrors), then the four row results by readlane.
template <bool kMax>
__device__ __forceinline__ uint32_t row_reduce(uint32_t v) {
  auto op = [](uint32_t x, uint32_t y) { return kMax ? max(x, y) : x + y; };
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x141, 0xF, 0xF, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x140, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_reduce<true>(v);
  return max(max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0)),
                 static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16))),
             max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32)),
                 static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48))));
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  const uint32_t r = row_reduce<false>(static_cast<uint32_t>(v));
  return __builtin_amdgcn_readlane(static_cast<int>(r), 0) + __builtin_amdgcn_readlane(static_cast<int>(r), 16) +
         __builtin_amdgcn_readlane(static_cast<int>(r), 32) + __builtin_amdgcn_readlane(static_cast<int>(r), 48);
}

// Rotated, split activations of one chunk of one batch row.
struct Split {
  uint32_t hi, lo;    // byte e: the int8 terms of element 64 g + 16 e + i of lane (g, i)
  float sigma;
  int sum_hi, sum_lo; // over the whole chunk
};

// Rotation and int8 split of one 256-chunk on one wave, on the matrix cores.
// With the chunk viewed as M[i][k] = x[16 i + k], H_256 x = H_16 M H_16 read
// row-major (H_256 = H_16 (x) H_16 in Sylvester order).  Lane (g, i) =
// (lane / 16, lane % 16) passes x[16 i + 4 g .. + 3] (bf16): one bf16 MFMA
// forms P = M H_16 (exact products, fp32 sums) and four fp32 MFMAs form
// H_16 P, which leaves element 64 g + 16 e + i in register e of lane (g, i).
__device__ __forceinline__ Split rotate_split(const uint2& xv, int lane) {
  const int g = lane >> 4, i = lane & 15;
  v4s a, hs;
  __builtin_memcpy(&a, &xv, 8);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) hs[kk] = static_cast<short>(hsign(4 * g + kk, i) < 0.0f ? 0xBF80 : 0x3F80);
  const v4f p = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, hs, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  v4f r = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) r = __builtin_amdgcn_mfma_f32_16x16x4f32(hsign(i, 4 * g + kk), p[kk], r, 0, 0, 0);
  uint32_t ab = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) ab = max(ab, __float_as_uint(r[e]) & 0x7fffffffu);
  const float amax = __uint_as_float(wave_max_u32(ab));
  Split sp;
  sp.sigma = amax * (1.0f / 127.0f);
  // |r| <= amax, so u = r / sigma lies in [-127, 127] up to the reciprocal's
  // rounding, and (u - hi) * 128 in [-64, 64]: no clamping is needed.  Adding
  // 1.5 * 2^23 rounds to the nearest integer (ties to even) and leaves it,
  // two's complement, in the low mantissa byte.
  const float rs = (amax > 0.0f) ? __builtin_amdgcn_rcpf(sp.sigma) : 0.0f;
  constexpr float kMagic = 12582912.0f;
  uint32_t hb[4], lb[4];
  float shf = 0.0f, slf = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float u = r[e] * rs;
    const float th = u + kMagic;
    const float hf = th - kMagic;
    const float tl = (u - hf) * 128.0f + kMagic;
    hb[e] = __float_as_uint(th);
    lb[e] = __float_as_uint(tl);
    shf += hf;
    slf += tl - kMagic;
  }
  // low bytes of the four words -> one word (byte e from word e)
  sp.hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(hb[3], hb[2], 0x0c0c0400u), __builtin_amdgcn_perm(hb[1], hb[0], 0x0c0c0400u), 0x05040100u);
  sp.lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(lb[3], lb[2], 0x0c0c0400u), __builtin_amdgcn_perm(lb[1], lb[0], 0x0c0c0400u), 0x05040100u);
  // both sums are within +-256 * 127, so one int32 carries them: 65536 sh + sl
  const int packed = wave_sum_i32(static_cast<int>(shf) * 65536 + static_cast<int>(slf));
  sp.sum_lo = static_cast<int>(static_cast<int16_t>(packed & 0xFFFF));
  sp.sum_hi = (packed - sp.sum_lo) / 65536;
  return sp;
}

// Pre-pass for batches above kFusedBatch: one wave per (chunk, batch row).
// act: [nv][4 t][4 g][batch][16] int8 a_hi (element 64 g + 16 t + p of the
// chunk at byte p), then (at + batch * d_in) a_lo, so that the operand load of
// one MFMA t reads 16 bytes per lane from one contiguous span;
// stats: [batch][nv] {sigma, sum a_hi, sum a_lo, 0} (the sums as int bits).
__global__ __launch_bounds__(64) void had256_prep_kernel(const uint16_t* __restrict__ x, int batch, int d_in,
                                                         int8_t* __restrict__ act, float4* __restrict__ stats) {
  const int lane = threadIdx.x, c = blockIdx.x, b = blockIdx.y;
  const int nv = d_in / kVec;
  const int g = lane >> 4, i = lane & 15;
  const uint2 xv =
      *reinterpret_cast<const uint2*>(x + static_cast<size_t>(b) * d_in + c * kVec + 16 * i + 4 * g);
  const Split sp = rotate_split(xv, lane);
  // element 64 g + 16 e + i is byte i of operand (t = e, g)
  const size_t lo_off = static_cast<size_t>(batch) * d_in;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const size_t o = ((static_cast<size_t>(c) * 16 + 4 * e + g) * batch + b) * 16 + i;
    act[o] = static_cast<int8_t>(sp.hi >> (8 * e));
    act[lo_off + o] = static_cast<int8_t>(sp.lo >> (8 * e));
  }
  if (lane == 0)
    stats[static_cast<size_t>(b) * nv + c] =
        make_float4(sp.sigma, __int_as_float(sp.sum_hi), __int_as_float(sp.sum_lo), 0.0f);
}

// Activation operands of one chunk for MFMA t = 0..3 (lane column n = r16 is
// batch row n), its sigma and the sums that undo the +4 code offset.
struct Act {
  v4i ah[4], al[4];
  float sg;
  int sum_hi, sum_lo;
};

// Lanes past the batch read row nb - 1 instead of zeros; their output columns
// are never stored.
__device__ __forceinline__ void load_act(const int8_t* __restrict__ act, const int8_t* __restrict__ act_lo,
                                         const float4* __restrict__ stats, int c, int nv, int nb, int r16, int g,
                                         Act& a) {
  const int n = min(r16, nb - 1);
  // 32-bit lane offsets: the operand planes are below 2^24 * 16 bytes
  const uint32_t o = ((static_cast<uint32_t>(c) * 16 + g) * nb + n) * 16;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a.ah[t] = *reinterpret_cast<const v4i*>(act + (o + 64 * t * nb));
    a.al[t] = *reinterpret_cast<const v4i*>(act_lo + (o + 64 * t * nb));
  }
  const float4 st = stats[static_cast<size_t>(n) * nv + c];
  a.sg = st.x;
  a.sum_hi = __float_as_int(st.y);
  a.sum_lo = __float_as_int(st.z);
}

// Operand dword i of MFMA t from the lane's record bytes: four stored codes
// c in [1, 7], bits 0-1 from low-plane dword i at bits 2 t of each byte, bit 2
// from high-plane dword i / 2 at bit 2 t + i % 2 of each byte.
template <int t, int i>
__device__ __forceinline__ int codes4(const uint4& p1, const uint2& p2) {
  const uint32_t d = (i == 0) ? p1.x : (i == 1) ? p1.y : (i == 2) ? p1.z : p1.w;
  const uint32_t e = (i < 2) ? p2.x : p2.y;
  constexpr int u = 2 * t + (i & 1);
  const uint32_t hb = (u >= 2) ? (e >> (u - 2)) : (e << (2 - u));
  return static_cast<int>(((d >> (2 * t)) & 0x03030303u) | (hb & 0x04040404u));
}

template <int t>
__device__ __forceinline__ v4i codes16(const uint4& p1, const uint2& p2) {
  return v4i{codes4<t, 0>(p1, p2), codes4<t, 1>(p1, p2), codes4<t, 2>(p1, p2), codes4<t, 3>(p1, p2)};
}

// One 16-row tile times one chunk; lane (r16, g) gets rows 4 g + e of the
// tile for batch column r16.  sc holds the rows' fp16 scales; f = sigma /
// 2048 folds in 1/16 for H and 1/128 for the a_lo weight, so that the exact
// int32 128 hi + lo (below 2^24, so exact in fp32) times s f is the term.
__device__ __forceinline__ void tile_dot(const uint4& p1, const uint2& p2, const uint2& sc, const Act& a, float f,
                                         float (&yp)[4]) {
  v4i dh = v4i{-4 * a.sum_hi, -4 * a.sum_hi, -4 * a.sum_hi, -4 * a.sum_hi};
  v4i dl = v4i{-4 * a.sum_lo, -4 * a.sum_lo, -4 * a.sum_lo, -4 * a.sum_lo};
  {
    const v4i w = codes16<0>(p1, p2);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.ah[0], dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.al[0], dl, 0, 0, 0);
  }
  {
    const v4i w = codes16<1>(p1, p2);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.ah[1], dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.al[1], dl, 0, 0, 0);
  }
  {
    const v4i w = codes16<2>(p1, p2);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.ah[2], dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.al[2], dl, 0, 0, 0);
  }
  {
    const v4i w = codes16<3>(p1, p2);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.ah[3], dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, a.al[3], dl, 0, 0, 0);
  }
  const uint32_t sw[2] = {sc.x, sc.y};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    _Float16 hs;
    const uint16_t sb = static_cast<uint16_t>(sw[e >> 1] >> (16 * (e & 1)));
    __builtin_memcpy(&hs, &sb, 2);
    const int d = dh[e] * 128 + dl[e];
    yp[e] = fmaf(static_cast<float>(hs), f * static_cast<float>(d), yp[e]);
  }
}

// One workgroup per 64 output rows (four 16-row blocks), 16 waves.  Wave w
// takes chunks w, w + 16, ...; per chunk it loads its four records' lane
// slices straight into registers (16 + 8 contiguous bytes per lane per
// record, so each load instruction reads one contiguous span) and runs all
// four tiles against each activation operand, so that an operand fetched
// once serves 64 rows.  With kFused the wave rotates and splits the chunk's
// activations itself from bf16 x (through a wave-private LDS slot);
// otherwise they come from the pre-pass.  The wave partial sums are added in
// LDS in a fixed order.
template <int B, bool kFused>
__global__ __launch_bounds__(64 * kGemvWaves) void had256_gemv_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ act, const float4* __restrict__ stats,
    const uint8_t* __restrict__ packed, float* __restrict__ y, int nb, int d_out, int d_in) {
  static_assert(!kFused || B <= kFusedBatch, "the in-kernel rotation serves up to kFusedBatch rows");
  // B is the compiled batch capacity; nb <= B rows of x / y are real.
  __shared__ __attribute__((aligned(16))) int8_t act_l[kFused ? kGemvWaves : 1][2][4][4][B][16];   // [.][hi/lo][g][t][n][p]
  __shared__ float sg_l[kFused && B > 1 ? kGemvWaves : 1][B];
  __shared__ int2 sum_l[kFused && B > 1 ? kGemvWaves : 1][B];
  __shared__ float red[kGemvWaves][kGemvRows][B];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: chunk addresses stay scalar
  const int r16 = lane & 15, g = lane >> 4;
  const int nv = d_in / kVec;
  const int nrb = (d_out + kBlockRows - 1) / kBlockRows;
  const int rb0 = blockIdx.x * kGemvTiles;
  const int8_t* act_lo = act + static_cast<size_t>(nb) * d_in;
  // the workgroup's records as one buffer: offsets fit 32 bits (d_in <= 2^24)
  const uint8_t* wg_rec = packed + static_cast<size_t>(rb0) * nv * kRecord;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wg_rec), 0, min(kGemvTiles, nrb - rb0) * nv * kRecord, 0x00020000);
  float yp[kGemvTiles][4];
#pragma unroll
  for (int T = 0; T < kGemvTiles; ++T) yp[T][0] = yp[T][1] = yp[T][2] = yp[T][3] = 0.0f;

  for (int c = wave; c < nv; c += kGemvWaves) {
    // Loads go out in the order they are consumed: the activations first,
    // then the records, so that each tile's work waits only for its own
    // record.  None is conditional (a conditional load makes every later
    // wait a full drain): blocks past the last re-read the last block, whose
    // outputs are never stored.
    Act a;
    uint2 xv[kFused ? B : 1];
    if constexpr (kFused) {
#pragma unroll
      for (int b = 0; b < B; ++b)   // rows past nb repeat row nb - 1
        xv[b] = *reinterpret_cast<const uint2*>(x + static_cast<size_t>(min(b, nb - 1)) * d_in + c * kVec + 16 * r16 +
                                                4 * g);
    } else {
      load_act(act, act_lo, stats, c, nv, nb, r16, g, a);
    }
    uint4 p1[kGemvTiles];
    uint2 p2[kGemvTiles], sc[kGemvTiles];
    // buffer loads: the record's offset is uniform (scalar), the three lane
    // offsets are the same for every record
#pragma unroll
    for (int T = 0; T < kGemvTiles; ++T) {
      const int so = (min(T, nrb - 1 - rb0) * nv + c) * kRecord;
      const v4i v1 = __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * lane, so, 0);
      const v2i v2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, kHiPlane + 8 * lane, so, 0);
      const v2i v3 = __builtin_amdgcn_raw_buffer_load_b64(rsrc, kScales + 8 * g, so, 0);
      p1[T] = make_uint4(v1.x, v1.y, v1.z, v1.w);
      p2[T] = make_uint2(v2.x, v2.y);
      sc[T] = make_uint2(v3.x, v3.y);
    }
    // keep every load above issued before any work that waits on one of them
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kFused) {
      Split sp0;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const Split sp = rotate_split(xv[b], lane);
        // element 64 g + 16 e + r16 of row b is byte r16 of operand (t = e, g), column b
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          act_l[wave][0][g][e][b][r16] = static_cast<int8_t>(sp.hi >> (8 * e));
          act_l[wave][1][g][e][b][r16] = static_cast<int8_t>(sp.lo >> (8 * e));
        }
        if constexpr (B == 1) {
          sp0 = sp;
        } else if (lane == 0) {   // sigma and the sums are wave-uniform
          sg_l[wave][b] = sp.sigma;
          sum_l[wave][b] = make_int2(sp.sum_hi, sp.sum_lo);
        }
      }
      wave_lds_sync();
      const int n = min(r16, nb - 1);   // lanes past the batch read row nb - 1; never stored
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a.ah[t] = *reinterpret_cast<const v4i*>(&act_l[wave][0][g][t][n][0]);
        a.al[t] = *reinterpret_cast<const v4i*>(&act_l[wave][1][g][t][n][0]);
      }
      if constexpr (B == 1) {
        a.sg = sp0.sigma;
        a.sum_hi = sp0.sum_hi;
        a.sum_lo = sp0.sum_lo;
      } else {
        a.sg = sg_l[wave][n];
        const int2 sm = sum_l[wave][n];
        a.sum_hi = sm.x;
        a.sum_lo = sm.y;
      }
    }
    const float f = a.sg * (1.0f / 2048.0f);
#pragma unroll
    for (int T = 0; T < kGemvTiles; ++T) tile_dot(p1[T], p2[T], sc[T], a, f, yp[T]);
    if constexpr (kFused) wave_lds_sync();   // this chunk's slot is read before the next chunk rewrites it
  }
  if (r16 < B) {
#pragma unroll
    for (int T = 0; T < kGemvTiles; ++T) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][16 * T + 4 * g + e][r16] = yp[T][e];
    }
  }
  __syncthreads();
  const int row0 = rb0 * kBlockRows;
  for (int i = tid; i < kGemvRows * B; i += 64 * kGemvWaves) {
    const int rl = i / B, b = i % B, orow = row0 + rl;
    if (b < nb && orow < d_out) {
      float sum = red[0][rl][b];
#pragma unroll
      for (int w = 1; w < kGemvWaves; ++w) sum += red[w][rl][b];
      y[static_cast<size_t>(b) * d_out + orow] = sum;
    }
  }
}

template <int B, bool kFused>
void launch_gemv(int nb, int d_out, int d_in, const uint16_t* x, const int8_t* act, const float4* stats,
                 const uint8_t* packed, float* y, hipStream_t s) {
  const int nrb = (d_out + kBlockRows - 1) / kBlockRows;
  hipLaunchKernelGGL((had256_gemv_kernel<B, kFused>), dim3((nrb + kGemvTiles - 1) / kGemvTiles),
                     dim3(64 * kGemvWaves), 0, s, x, act, stats, packed, y, nb, d_out, d_in);
}

}  // namespace

extern "C" {

size_t wush_had256_packed_bytes(int d_out, int d_in) {
  if (d_out < 0 || d_in < kVec || d_in % kVec) return 0;
  return static_cast<size_t>((d_out + kBlockRows - 1) / kBlockRows) * (d_in / kVec) * kRecord;
}

wush_status wush_had256_pack_weights(int d_out, int d_in, const float* W, uint8_t* packed, void* stream) {
  if (d_out < 0 || d_in < kVec || d_in % kVec)
    return wush::fail(WUSH_E_SHAPE, "wush_had256_pack_weights: d_in must be a positive multiple of 256");
  if (d_out == 0) return WUSH_OK;
  if (!W || !packed) return wush::fail(WUSH_E_ARG, "wush_had256_pack_weights: null pointer");
  if (!wush::aligned16(packed)) return wush::fail(WUSH_E_ARG, "wush_had256_pack_weights: packed must be 16-byte aligned");
  const size_t rows = static_cast<size_t>((d_out + kBlockRows - 1) / kBlockRows) * kBlockRows;
  const size_t nvec = rows * (d_in / kVec);
  if (nvec > 0x7fffffffu) return wush::fail(WUSH_E_SHAPE, "wush_had256_pack_weights: too many vectors");
  hipLaunchKernelGGL(had256_pack_kernel, dim3(static_cast<unsigned>(nvec)), dim3(kVec), 0,
                     static_cast<hipStream_t>(stream), W, d_out, d_in, packed);
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

size_t wush_had256_gemv_ws_bytes(int batch, int d_in) {
  if (batch < 1 || d_in < kVec || d_in % kVec) return 0;
  if (batch <= kFusedBatch) return 0;                                 // rotated inside the GEMV
  const size_t act = 2 * static_cast<size_t>(batch) * d_in;           // a_hi, a_lo
  return act + static_cast<size_t>(batch) * (d_in / kVec) * sizeof(float4);   // sigma and sums
}

wush_status wush_had256_gemv(int batch, int d_out, int d_in, const uint16_t* x, const uint8_t* packed, float* y,
                             void* ws, size_t ws_bytes, void* stream) {
  if (batch < 1 || batch > 16 || d_out < 1 || d_in < kVec || d_in % kVec || d_in > (1 << 24))
    return wush::fail(WUSH_E_SHAPE, "wush_had256_gemv: need 1 <= batch <= 16, d_out >= 1, d_in %% 256 == 0, d_in <= 2^24");
  if (!x || !packed || !y) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: null pointer");
  if (!wush::aligned16(packed) || !wush::aligned16(x))
    return wush::fail(WUSH_E_ARG, "wush_had256_gemv: x and packed must be 16-byte aligned");
  if (ws && !wush::aligned16(ws)) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch <= kFusedBatch) {
    if (batch == 1)
      launch_gemv<1, true>(batch, d_out, d_in, x, nullptr, nullptr, packed, y, s);
    else
      launch_gemv<kFusedBatch, true>(batch, d_out, d_in, x, nullptr, nullptr, packed, y, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_gemv launch: %s", hipGetErrorString(e));
    return WUSH_OK;
  }
  // rotated, int8-split activations: the caller's workspace, else stream-ordered scratch
  const int nv = d_in / kVec;
  const size_t act_bytes = 2 * static_cast<size_t>(batch) * d_in;
  const size_t need = wush_had256_gemv_ws_bytes(batch, d_in);
  uint8_t* wsp = static_cast<uint8_t*>(ws);
  if (wsp) {
    if (ws_bytes < need) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: workspace of %zu bytes, need %zu", ws_bytes, need);
  } else {
    const hipError_t ae = hipMallocAsync(reinterpret_cast<void**>(&wsp), need, s);
    if (ae != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_gemv scratch (%zu bytes): %s", need, hipGetErrorString(ae));
  }
  int8_t* act = reinterpret_cast<int8_t*>(wsp);
  float4* stats = reinterpret_cast<float4*>(wsp + act_bytes);
  hipLaunchKernelGGL(had256_prep_kernel, dim3(nv, batch), dim3(64), 0, s, x, batch, d_in, act, stats);
  launch_gemv<16, false>(batch, d_out, d_in, x, act, stats, packed, y, s);
  const hipError_t fe = ws ? hipSuccess : hipFreeAsync(wsp, s);
  if (fe != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_gemv scratch free: %s", hipGetErrorString(fe));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_gemv launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // extern "C"
