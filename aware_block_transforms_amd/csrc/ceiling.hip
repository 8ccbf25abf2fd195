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

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kAcc16 = 8;   // independent 16x16 accumulators per wave
constexpr int kAcc32 = 4;   // independent 32x32 accumulators per wave

// The MFMAs are inline asm with each accumulator tied to its own AGPR tuple:
// with the builtins the register allocator shuffles accumulators between
// tuples inside the loop (v_accvgpr moves), which is not the instruction's
// rate.  Operands are written long before the loop; the accumulators are read
// after 64 wait states.
template <bool BIG>
__global__ __launch_bounds__(256, 1) void fp4_stream(const uint32_t* __restrict__ bits, float* __restrict__ out,
                                                      int iters) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t* p = bits + (t & 1023) * 16;
  v4i a = {static_cast<int>(p[0]), static_cast<int>(p[1]), static_cast<int>(p[2]), static_cast<int>(p[3])};
  v4i b = {static_cast<int>(p[4]), static_cast<int>(p[5]), static_cast<int>(p[6]), static_cast<int>(p[7])};
  const int sa = static_cast<int>(p[8] & 0x7f7f7f7fu) | 0x40404040, sb = static_cast<int>(p[9] & 0x7f7f7f7fu) | 0x40404040;
  float sum = 0.0f;
  asm volatile("s_nop 7" ::: "memory");
  if constexpr (!BIG) {
    v4f acc[kAcc16];
#pragma unroll
    for (int i = 0; i < kAcc16; ++i) {
      acc[i] = v4f{static_cast<float>(i), 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[i]));
    }
    asm volatile("s_nop 7" ::: "memory");
    int it = 0;
    do {
#pragma unroll
      for (int i = 0; i < kAcc16; ++i)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+a"(acc[i]) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    } while (++it < iters);
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
    for (int i = 0; i < kAcc16; ++i) sum += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  } else {
    v16f acc[kAcc32];
#pragma unroll
    for (int i = 0; i < kAcc32; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] = e ? 0.0f : static_cast<float>(i);
      asm volatile("" : "+a"(acc[i]));
    }
    asm volatile("s_nop 7" ::: "memory");
    int it = 0;
    do {
#pragma unroll
      for (int i = 0; i < kAcc32; ++i)
        asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+a"(acc[i]) : "v"(a), "v"(b), "v"(sa), "v"(sb));
    } while (++it < iters);
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
    for (int i = 0; i < kAcc32; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[i][e];
  }
  out[t] = sum;
}

// The same instruction with operands that change from one MFMA to the next, in
// the W4A4 matmul's order: for each of 8 A operand sets, the 8 B sets into 8
// accumulators (B changes every MFMA, A every eighth), each set with its own
// random scale bytes.  A matmul feeds new operand bits to every MFMA, which
// the repeated-operand stream above does not.
__global__ __launch_bounds__(256, 1) void fp4_stream_vary(const uint32_t* __restrict__ bits, float* __restrict__ out,
                                                         int iters) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  v4i a[8], b[8];
  int sa[8], sb[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t* p = bits + ((t + 37 * c) & 1023) * 16;
    const uint32_t* q = bits + ((t + 101 * c + 500) & 1023) * 16;
    a[c] = v4i{static_cast<int>(p[0]), static_cast<int>(p[1]), static_cast<int>(p[2]), static_cast<int>(p[3])};
    b[c] = v4i{static_cast<int>(q[4]), static_cast<int>(q[5]), static_cast<int>(q[6]), static_cast<int>(q[7])};
    sa[c] = static_cast<int>(p[8] & 0x7f7f7f7fu) | 0x40404040;
    sb[c] = static_cast<int>(q[9] & 0x7f7f7f7fu) | 0x40404040;
  }
  float sum = 0.0f;
  v4f acc[kAcc16];
#pragma unroll
  for (int i = 0; i < kAcc16; ++i) {
    acc[i] = v4f{static_cast<float>(i), 0.f, 0.f, 0.f};
    asm volatile("" : "+a"(acc[i]));
  }
  asm volatile("s_nop 7" ::: "memory");
  int it = 0;
  do {
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < kAcc16; ++i)
        asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                     : "+a"(acc[i]) : "v"(b[i]), "v"(a[q]), "v"(sb[i]), "v"(sa[q]));
  } while (++it < iters);
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < kAcc16; ++i) sum += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
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

// HBM read rates of two access patterns over the same bytes (rows x row_bytes,
// row_bytes a multiple of 512), each lane folding its loads into one word:
//  * flat: each wave reads 4 KB contiguous pieces (one 1 KB load instruction
//    after another), pieces dealt round-robin over the waves;
//  * tiles: the transform step's pattern: a wave owns 128 contiguous bytes of
//    every row (its two 32-channel bf16 spans) and walks 16-row tiles, one
//    load instruction = 16 rows x 64 bytes, `depth` tiles in flight.
__global__ __launch_bounds__(256) void read_flat(const uint4* __restrict__ src, size_t n16, uint32_t* __restrict__ out) {
  const size_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6, waves = (gridDim.x * blockDim.x) >> 6;
  const int lane = threadIdx.x & 63;
  uint32_t acc = 0;
  for (size_t p = wave * 256; p < n16; p += waves * 256) {
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p + i * 64 + lane < n16 ? src[p + i * 64 + lane] : uint4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void read_tiles(const uint8_t* __restrict__ src, int rows, int row_bytes, int tiles_per_wave,
                                                  uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, q = lane >> 4;
  const int col = (blockIdx.x * 4 + wave) * 128;
  uint32_t acc = 0;
  if (col < row_bytes) {
    const int t0 = blockIdx.y * tiles_per_wave;
    for (int t = 0; t < tiles_per_wave; ++t) {
      const int row = min((t0 + t) * 16 + j, rows - 1);
      const uint8_t* p = src + static_cast<size_t>(row) * row_bytes + col + 16 * q;
      const uint4 a = *reinterpret_cast<const uint4*>(p), b = *reinterpret_cast<const uint4*>(p + 64);
      acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    }
  }
  out[(blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

template <typename K, typename... A>
int launch(K k, int blocks, void* stream, A... args) {
  hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), args...);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

// which: 0 = 16x16x128, 1 = 32x32x64, 2 = 16x16x128 with operands that change
// every MFMA (64 per iteration).  bits: >= 1024 * 16 uint32 of operand
// bits; out: blocks * 256 floats.  Returns 0 on a successful launch.
int wush_ceiling_fp4(int which, int blocks, int iters, const uint32_t* bits, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !bits || !out) return 1;
  if (which == 2) return launch(fp4_stream_vary, blocks, stream, bits, out, iters);
  return which ? launch(fp4_stream<true>, blocks, stream, bits, out, iters)
               : launch(fp4_stream<false>, blocks, stream, bits, out, iters);
}

// Read rates: pattern 0 = flat (grid of `blocks` workgroups), 1 = tiles
// (tiles_per_wave 16-row tiles per wave).  out: enough uint32 for the grid.
int wush_ceiling_read(int pattern, const void* src, int rows, int row_bytes, int blocks, int tiles_per_wave,
                      uint32_t* out, void* stream) {
  if (!src || !out || rows < 16 || row_bytes < 512 || row_bytes % 512) return 1;
  if (pattern == 0)
    return launch(read_flat, blocks, stream, static_cast<const uint4*>(src),
                  static_cast<size_t>(rows) * row_bytes / 16, out);
  if (tiles_per_wave < 1) return 1;
  const int gy = (rows / 16 + tiles_per_wave - 1) / tiles_per_wave;
  hipLaunchKernelGGL(read_tiles, dim3(row_bytes / 512, gy), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(src), rows, row_bytes, tiles_per_wave, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
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
