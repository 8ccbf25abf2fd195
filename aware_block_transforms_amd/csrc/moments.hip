// Calibration second moments on the GPU: Sx[b] = X_b^T X_b / n per block of
// bs channels.
//
// WUSH news article, deployment paragraph: the transforms are built from
// second moments of the activations, taken from calibration data, and the
// per-block work can run in parallel.  This is the step before the builder.
//
// One wave per (block, token chunk).  The chunk's rows of the block are
// staged in LDS 128 tokens at a time (fp32, 16 KB at bs 32, so that every
// wave of the grid is resident at once), with every load of a stage issued
// before the first is used (one memory round trip per stage).  The block's moment is then a [bs x tokens] x [tokens x bs] product
// on the fp64 matrix cores: v_mfma_f64_16x16x4 takes four tokens per step,
// one MFMA per 16 x 16 tile (three at bs 32: the two diagonal tiles and one
// off-diagonal tile, mirrored on output).  The product of two fp32 values is
// exact in fp64, so only the sums round.  Each value is written at (i, j) and
// (j, i) from one lane, so Sx is exactly symmetric.  A second kernel adds the
// chunk partials in chunk order, divides by n and rounds once to fp32.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "common.h"

namespace {

constexpr int kMomTokens = 256;   // tokens per chunk, while the chunk count stays at most kMaxChunks
constexpr int kMaxChunks = 64;
constexpr int kStage = 128;       // tokens staged in LDS at a time

typedef double v4d __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_at(uint32_t w, int half) { return __uint_as_float(half ? (w & 0xffff0000u) : (w << 16)); }

template <int BS, bool BF16>
__global__ __launch_bounds__(64) void moments_partial(const void* __restrict__ X, int n, int d_in, int per_chunk,
                                                      double* __restrict__ part) {
  constexpr int kElem = BF16 ? 2 : 4;
  constexpr int kRow = BS * kElem;                 // bytes of one token's block
  constexpr int kPieces = kStage * kRow / 16;      // 16-byte pieces of a stage
  static_assert(kPieces % 64 == 0, "whole pieces per lane");
  constexpr int kPer = 16 / kElem;                 // values per 16-byte piece
  __shared__ __attribute__((aligned(16))) float rows[kStage * BS];    // fp32 (exact for bf16 input); 16 KB at bs 32
  const int lane = threadIdx.x;
  const int b = blockIdx.x, ch = blockIdx.y, nblk = gridDim.x;
  const int t0 = ch * per_chunk, t1 = min(n, t0 + per_chunk);
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(X) + static_cast<size_t>(b) * kRow;
  const size_t stride = static_cast<size_t>(d_in) * kElem;
  v4d c00 = v4d{0.0, 0.0, 0.0, 0.0}, c01 = c00, c11 = c00;
  const int r16 = lane & 15, g = lane >> 4;
  for (int s0 = t0; s0 < t1; s0 += kStage) {
    const int rows_here = min(kStage, t1 - s0);
    // all of the stage's loads go out before the first is used: piece
    // lane + 64 k is bytes 16 (piece % (kRow/16)) of row piece / (kRow/16)
    uint4 v[kPieces / 64];
#pragma unroll
    for (int k = 0; k < kPieces / 64; ++k) {
      const int piece = lane + 64 * k, r = piece / (kRow / 16), part16 = piece % (kRow / 16);
      v[k] = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows_here) v[k] = *reinterpret_cast<const uint4*>(xb + (s0 + r) * stride + part16 * 16);
    }
#pragma unroll
    for (int k = 0; k < kPieces / 64; ++k) {
      const int piece = lane + 64 * k;
      float* d = rows + piece * kPer;              // piece order is row-major value order
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int e = 0; e < kPer; ++e) d[e] = BF16 ? bf16_at(w[e >> 1], e & 1) : __uint_as_float(w[e]);
    }
    __syncthreads();
    // four tokens per fp64 MFMA step (rows past rows_here hold zeros): lane
    // (g, r16) supplies token r + g, channel r16 (and 16 + r16) as both the
    // A operand (row index) and the B operand (column index)
    for (int r = 0; r < rows_here; r += 4) {
      const double a0 = static_cast<double>(rows[(r + g) * BS + r16]);
      c00 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, a0, c00, 0, 0, 0);
      if constexpr (BS == 32) {
        const double a1 = static_cast<double>(rows[(r + g) * BS + 16 + r16]);
        c01 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, a1, c01, 0, 0, 0);
        c11 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, a1, c11, 0, 0, 0);
      }
    }
    __syncthreads();   // the stage is read before the next one overwrites it
  }
  // the fp64 MFMA leaves row g + 4 e, column r16 of each 16 x 16 tile in
  // register e of lane (g, r16) (a GPU probe of the instruction's layout);
  // every value is written at (i, j) and (j, i) from one lane, so Sx is
  // exactly symmetric
  double* dst = part + (static_cast<size_t>(ch) * nblk + b) * BS * BS;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = g + 4 * e, j = r16;
    if (i <= j) {
      dst[i * BS + j] = c00[e];
      dst[j * BS + i] = c00[e];
      if constexpr (BS == 32) {
        dst[(16 + i) * BS + 16 + j] = c11[e];
        dst[(16 + j) * BS + 16 + i] = c11[e];
      }
    }
    if constexpr (BS == 32) {
      dst[i * BS + 16 + j] = c01[e];
      dst[(16 + j) * BS + i] = c01[e];
    }
  }
}

__global__ __launch_bounds__(256) void moments_reduce(const double* __restrict__ part, int chunks, size_t elems, int n,
                                                      float* __restrict__ Sx) {
  const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= elems) return;
  double s = 0.0;
  for (int c = 0; c < chunks; ++c) s += part[static_cast<size_t>(c) * elems + e];
  Sx[e] = static_cast<float>(s / n);
}

int chunk_count(int n) { return std::min(kMaxChunks, (n + kMomTokens - 1) / kMomTokens); }

}  // namespace

extern "C" {

size_t wush_block_moments_dev_ws_bytes(int bs, int n, int d_in) {
  if ((bs != 16 && bs != 32) || n < 1 || d_in < bs || d_in % bs) return 0;
  return static_cast<size_t>(chunk_count(n)) * d_in * bs * sizeof(double);
}

wush_status wush_block_moments_dev(int bs, wush_dtype xdt, int n, int d_in, const void* X, float* Sx, void* ws,
                                   size_t ws_bytes, void* stream) {
  WUSH_REQUIRE(bs == 16 || bs == 32, WUSH_E_SHAPE, "wush_block_moments_dev: bs must be 16 or 32 (got %d)", bs);
  WUSH_REQUIRE(n >= 1 && d_in >= bs && d_in % bs == 0, WUSH_E_SHAPE,
               "wush_block_moments_dev: need n >= 1 and d_in %% bs == 0 (n=%d d_in=%d bs=%d)", n, d_in, bs);
  WUSH_REQUIRE(X && Sx, WUSH_E_ARG, "wush_block_moments_dev: null pointer");
  WUSH_REQUIRE(xdt == WUSH_F32 || xdt == WUSH_BF16, WUSH_E_ARG, "wush_block_moments_dev: bad dtype");
  WUSH_REQUIRE(wush::aligned16(X), WUSH_E_ARG, "wush_block_moments_dev: X must be 16-byte aligned");
  WUSH_REQUIRE(!ws || wush::aligned16(ws), WUSH_E_ARG, "wush_block_moments_dev: workspace must be 16-byte aligned");
  const int nblk = d_in / bs;
  WUSH_REQUIRE(nblk <= 2147483647 / 64, WUSH_E_SHAPE, "wush_block_moments_dev: too many blocks");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = wush_block_moments_dev_ws_bytes(bs, n, d_in);
  double* part = static_cast<double*>(ws);
  if (part) {
    WUSH_REQUIRE(ws_bytes >= need, WUSH_E_ARG, "wush_block_moments_dev: workspace of %zu bytes, need %zu", ws_bytes,
                 need);
  } else {
    const hipError_t ae = hipMallocAsync(reinterpret_cast<void**>(&part), need, s);
    if (ae != hipSuccess)
      return wush::fail(WUSH_E_HIP, "wush_block_moments_dev scratch (%zu bytes): %s", need, hipGetErrorString(ae));
  }
  const int chunks = chunk_count(n);
  const int per_chunk = (n + chunks - 1) / chunks;
  const bool bf16 = xdt == WUSH_BF16;
  const dim3 grid(nblk, chunks);
  if (bs == 32) {
    if (bf16) hipLaunchKernelGGL((moments_partial<32, true>), grid, dim3(64), 0, s, X, n, d_in, per_chunk, part);
    else hipLaunchKernelGGL((moments_partial<32, false>), grid, dim3(64), 0, s, X, n, d_in, per_chunk, part);
  } else {
    if (bf16) hipLaunchKernelGGL((moments_partial<16, true>), grid, dim3(64), 0, s, X, n, d_in, per_chunk, part);
    else hipLaunchKernelGGL((moments_partial<16, false>), grid, dim3(64), 0, s, X, n, d_in, per_chunk, part);
  }
  const size_t elems = static_cast<size_t>(nblk) * bs * bs;
  hipLaunchKernelGGL(moments_reduce, dim3(static_cast<unsigned>((elems + 255) / 256)), dim3(256), 0, s, part, chunks,
                     elems, n, Sx);
  const hipError_t e = hipGetLastError();
  const hipError_t f = ws ? hipSuccess : hipFreeAsync(part, s);
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_block_moments_dev launch: %s", hipGetErrorString(e));
  if (f != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_block_moments_dev scratch free: %s", hipGetErrorString(f));
  return WUSH_OK;
}

}  // extern "C"
