// INT4 x INT4 -> fp32 matmul for gfx950, LDS-staged.
//
// WUSH news article (chain.bitekongjian.com), experiments paragraph: the
// format sweep includes INT4 (symmetric codes in [-7, 7], one fp16 scale per
// 32 values).  A dequantized value q s needs up to 14 significant bits, more
// than fp16 holds, so the codes stay integers: each 32-group is one int8
// MFMA (v_mfma_i32_16x16x32_i8) into a fresh int32, which is exact, and the
// group's two scales multiply that sum in fp32 (s_a s_b has at most 22
// significant bits, so only the final fma rounds) into fp32 accumulators.
// The per-group rescale (convert, multiply, fma per output) is vector-ALU
// work on every output for every 32 of K and bounds the kernel; the matrix
// cores are idle most of the time.
//
// Decode: a nibble placed in the high half of a byte is the int8 16 q, so
// one shift-and-mask per four values feeds the MFMA; the factor 256 it puts on
// each product is folded into the weight scales by the pre-pass (a power of
// two, exact).
//
// Tile: 256 (activation rows) x 128 (weight rows) per workgroup, eight waves
// (two per SIMD) of 64 x 64: 64 fp32 accumulators per lane in VGPRs, where the
// rescale can reach them, and room for the MFMA results to land in VGPRs
// too; K in blocks of 256 (8 groups) staged through two LDS buffers by
// buffer_load ... lds one block ahead.  The pre-pass re-lays the scales as
// fp32 so that a wave's reads are broadcasts.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBM = 256, kBN = 128;
constexpr int kCodeA = kBM * 128, kCodeB = kBN * 128;   // codes of one block: rows x 128 B
constexpr int kScaleA = kBM * 8 * 4, kScaleB = kBN * 8 * 4;   // fp32 scales of one block: rows x 8 groups
constexpr int kStageBytes = kCodeA + kCodeB + kScaleA + kScaleB;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;
constexpr unsigned kWaitLgkm0 = 0xC07F;   // s_waitcnt lgkmcnt(0) (gfx9 layout)
constexpr unsigned kWaitVm0 = 0x0F70;     // s_waitcnt vmcnt(0)

// Raw buffer descriptor: base address, stride 0, `bytes` records; dword 3 =
// 0x00020000 selects the 32-bit data format for untyped access on CDNA.
__device__ __forceinline__ v4i make_desc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return v4i{static_cast<int>(static_cast<uint32_t>(b)), static_cast<int>((b >> 32) & 0xFFFFu),
             static_cast<int>(bytes), 0x00020000};
}

// 16 bytes per lane from buffer `desc` at byte voff + soff (zeros where that
// is at or past its end) straight into LDS at lds + 16 lane (buffer_load ...
// lds; lds is wave-uniform).  Written as asm so that the compiler does not
// treat it as an LDS store and make every later LDS read wait for all DMA in
// flight; the kernel orders the two itself (s_waitcnt vmcnt(0) and a barrier
// before LDS written by DMA is read).  The instruction writes no register
// except M0, which nothing else in these kernels reads (a CPU test checks the
// compiled code).
__device__ __forceinline__ void dma16(const v4i& desc, const void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
}

// All of this wave's LDS reads done, then the workgroup barrier.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XCD-aware tile order: workgroups are dealt to the 8 XCDs round-robin, each
// XCD gets a contiguous run of tiles walked in groups of kGroupM tile rows.
__device__ __forceinline__ void tile_of(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = id % kXcds, local = id / kXcds;
  const int linear = xcd * per + min(xcd, rem) + local;
  const int width = kGroupM * tiles_n;
  const int group = linear / width;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = linear - group * width;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// Scales re-laid as fp32 (exact), per tile and 256-wide K block (groups
// g = 0..7 of it; zero past K and past the operand):
//   activation tile (256 rows, row 64 w + 16 q + r):  float ((g 4 + w) 16 + r) 4 + q
//   weight tile (128 rows, row 64 w + 16 i + 4 c + e):  float ((g 2 + w) 4 + c) 16 + 4 i + e,
//   times 1/256 (the decode's 16 q on both sides).
// So a lane reads its four activation scales, or its sixteen weight scales,
// of a group as contiguous fp32 that lanes sharing them read at the same
// address.  Grid (K blocks, tiles_a + tiles_b), 256 threads (thread = tile row).
__global__ __launch_bounds__(256) void int4_scales_to_planes(const uint16_t* __restrict__ SA, int ra,
                                                             const uint16_t* __restrict__ SB, int rb, int tiles_a,
                                                             int K, int nb, uint8_t* __restrict__ PA,
                                                             uint8_t* __restrict__ PB) {
  __shared__ __attribute__((aligned(16))) float planes[kBM * 8];
  const int k = blockIdx.x, t = blockIdx.y, tr = threadIdx.x;
  const bool in_a = t < tiles_a;
  const int tile_rows = in_a ? kBM : kBN;
  const int row = (in_a ? t : t - tiles_a) * tile_rows + tr;
  const int rows = in_a ? ra : rb;
  const int spr = K / 32;   // scales per row
  if (tr < tile_rows) {
    const uint16_t* s = (in_a ? SA : SB) + static_cast<size_t>(min(row, rows - 1)) * spr;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int idx = 8 * k + g;
      float v = (row < rows && idx < spr) ? f16_to_f32(s[idx]) : 0.0f;
      int pos;
      if (in_a) {
        const int w = tr >> 6, q = (tr >> 4) & 3, r = tr & 15;
        pos = ((g * 4 + w) * 16 + r) * 4 + q;
      } else {
        const int w = tr >> 6, i = (tr >> 4) & 3, c = (tr >> 2) & 3, e = tr & 3;
        pos = ((g * 2 + w) * 4 + c) * 16 + 4 * i + e;
        v *= 0.00390625f;
      }
      planes[pos] = v;
    }
  }
  __syncthreads();
  const int bytes = tile_rows * 8 * 4;
  uint8_t* dst = (in_a ? PA + (static_cast<size_t>(t) * nb + k) * kScaleA
                       : PB + (static_cast<size_t>(t - tiles_a) * nb + k) * kScaleB);
  for (int o = tr * 16; o < bytes; o += 256 * 16)
    *reinterpret_cast<uint4*>(dst + o) = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(planes) + o);
}

struct Ctx {
  v4i ra, rb, rsa, rsb;
  uint32_t dma_off[2];           // loader lane's offset within 8 rows x 128 B, for even / odd u
  uint32_t a_row0, b_row0;       // byte offset of the wave's first loaded row of A (32 rows) and B (16 rows)
  uint32_t krow;
  uint32_t sa_base, sb_base;     // byte offset of the tile's re-laid scales (block 0)
  uint32_t r_base, r_sw16;       // read lane: rr * 128 + 4 grp, and 16 ((rr / 2) % 8)
  uint32_t r_sa, r_sb;           // LDS offsets of this lane's scales for group 0
  int wave, wm, wn;
};

// DMA d (0..7) of this wave's share of block kb into stage `buf`: d < 4: A
// codes rows 32 wave + 8 d .. + 7; d < 6: B codes rows 16 wave + 8 (d - 4)
// .. + 7; 6: this wave's 1 KB of A's scales; 7: 1 KB of B's (waves 0-3).  Each
// lane fetches the global chunk that the XOR swizzle (chunk c of row R in
// slot c ^ ((R / 2) % 8)) puts in its slot.  Rows past the operand read as
// zeros; in a half block the upper 64 bytes of a row read the next row or
// zeros, multiplied by the zero scales past K.
__device__ __forceinline__ void dma(const Ctx& c, int d, int kb, uint8_t* buf) {
  const int lane = threadIdx.x & 63;
  const uint32_t kofs = static_cast<uint32_t>(kb) * 128;
  if (d < 4) {
    dma16(c.ra, buf + c.wave * (32 * 128) + d * 1024, c.dma_off[d & 1],
          c.a_row0 + static_cast<uint32_t>(8 * d) * c.krow + kofs);
  } else if (d < 6) {
    const int u = d - 4;
    dma16(c.rb, buf + kCodeA + c.wave * (16 * 128) + u * 1024, c.dma_off[u & 1],
          c.b_row0 + static_cast<uint32_t>(8 * u) * c.krow + kofs);
  } else if (d == 6) {
    dma16(c.rsa, buf + kCodeA + kCodeB + c.wave * 1024, lane * 16,
          c.sa_base + static_cast<uint32_t>(kb) * kScaleA + c.wave * 1024);
  } else if (c.wave < 4) {
    dma16(c.rsb, buf + kCodeA + kCodeB + kScaleA + c.wave * 1024, lane * 16,
          c.sb_base + static_cast<uint32_t>(kb) * kScaleB + c.wave * 1024);
  }
}

// nibbles of w (element 2 i in the low nibble of byte i) as int8 16 q, in
// the K order [0 2 4 6 1 3 5 7] (the same on both operands)
__device__ __forceinline__ long widen16(uint32_t w) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u, hi = w & 0xF0F0F0F0u;
  return static_cast<long>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Raw operand dwords and scales of one group.
struct Group {
  uint32_t a[4], b[4];
  v4f sa;         // activation scales of m fragments 0..3
  v4f sb[4];      // weight scales (x 1/256) of n fragment i, rows 4 c + 0..3
};

__device__ __forceinline__ void read_group(const Ctx& c, const uint8_t* buf, int g, Group& G) {
  const uint32_t off = c.r_base + ((16u * g) ^ c.r_sw16);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    G.a[q] = *reinterpret_cast<const uint32_t*>(buf + (64 * c.wm + 16 * q) * 128 + off);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    G.b[i] = *reinterpret_cast<const uint32_t*>(buf + kCodeA + (64 * c.wn + 16 * i) * 128 + off);
  G.sa = *reinterpret_cast<const v4f*>(buf + kCodeA + kCodeB + c.r_sa + g * (4 * 16 * 4 * 4));
  const uint8_t* sb = buf + kCodeA + kCodeB + kScaleA + c.r_sb + g * (2 * 4 * 16 * 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) G.sb[i] = *reinterpret_cast<const v4f*>(sb + 16 * i);
}

// acc[q][i][e] += sum over the group of A[m][k] B[n][k], m = 64 wm + 16 q + rr,
// n = 64 wn + 16 i + 4 grp + e.  The group's 16 MFMAs are issued before its
// rescale, so the rescale reads finished results instead of waiting on each
// MFMA in turn (half the hazard padding; 443-447 against 473-475 us on the
// 4096 x 4096 layer at 8192 tokens).  Each output still takes one fma per
// group, groups in order.
__device__ __forceinline__ void compute_group(const Group& G, float (&acc)[4][4][4]) {
  long a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) a[q] = widen16(G.a[q]);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = widen16(G.b[i]);
  v4i p[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) p[q][i] = __builtin_amdgcn_mfma_i32_16x16x32_i8(b[i], a[q], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float sa = G.sa[q];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[q][i][e] = __builtin_fmaf(static_cast<float>(p[q][i][e]) * G.sb[i][e], sa, acc[q][i][e]);
  }
}

__global__ __launch_bounds__(512, 1) void gemm_int4_lds(const uint8_t* __restrict__ A, const uint8_t* __restrict__ PA,
                                                       const uint8_t* __restrict__ B, const uint8_t* __restrict__ PB,
                                                       float* __restrict__ Y, int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];
  Ctx c;
  const int tid = threadIdx.x, lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.wm = c.wave >> 1;   // 0..3: activation rows 64 wm ..
  c.wn = c.wave & 1;    // 0..1: weight rows 64 wn ..
  const int nb = (K + 255) / 256;
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int rr = lane & 15, grp = lane >> 4;
  c.krow = static_cast<uint32_t>(K) / 2;   // the host checks the operands are below 2^31 bytes
  const int lr = lane >> 3, lc = lane & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    c.dma_off[h] = static_cast<uint32_t>(lr) * c.krow + ((lc ^ (((lr + 8 * h) >> 1) & 7)) * 16);
  c.a_row0 = static_cast<uint32_t>(m0 + 32 * c.wave) * c.krow;
  c.b_row0 = static_cast<uint32_t>(n0 + 16 * c.wave) * c.krow;
  c.sa_base = static_cast<uint32_t>(tm * nb) * kScaleA;
  c.sb_base = static_cast<uint32_t>(tn * nb) * kScaleB;
  // fragment rows are 16-aligned, so row R's swizzle is (rr / 2) % 8
  c.r_base = rr * 128 + 4 * grp;
  c.r_sw16 = 16 * ((rr >> 1) & 7);
  c.r_sa = ((c.wm * 16) + rr) * 4 * 4;
  c.r_sb = ((c.wn * 4) + grp) * 16 * 4;
  c.ra = make_desc(A, static_cast<uint32_t>(M) * c.krow);
  c.rb = make_desc(B, static_cast<uint32_t>(N) * c.krow);
  c.rsa = make_desc(PA, static_cast<uint32_t>(tiles_m * nb) * kScaleA);
  c.rsb = make_desc(PB, static_cast<uint32_t>(tiles_n * nb) * kScaleB);

  float acc[4][4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[q][i][e] = 0.0f;

  uint8_t* const buf0 = smem;
  uint8_t* const buf1 = smem + kStageBytes;
#pragma unroll
  for (int d = 0; d < 8; ++d) dma(c, d, 0, buf0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  stage_barrier();
  int k = 0;
#pragma unroll 1
  do {
    uint8_t* cur = (k & 1) ? buf1 : buf0;
    uint8_t* nxt = (k & 1) ? buf0 : buf1;
    // block k + 1 into the buffer block k - 1 used (every wave has passed the
    // barrier that ended block k - 1); past the last block, the last block
    // again (no branch)
#pragma unroll
    for (int d = 0; d < 8; ++d) dma(c, d, min(k + 1, nb - 1), nxt);
    Group G[2];
    read_group(c, cur, 0, G[0]);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < 7) read_group(c, cur, g + 1, G[(g + 1) & 1]);
      compute_group(G[g & 1], acc);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stage_barrier();
    ++k;
  } while (k < nb);

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = m0 + 64 * c.wm + 16 * q + rr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 64 * c.wn + 16 * i + 4 * grp;
      float* dst = Y + static_cast<size_t>(m) * N + n;
      if (n + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[q][i][0], acc[q][i][1], acc[q][i][2], acc[q][i][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) dst[e] = acc[q][i][e];
      }
    }
  }
}

bool use_int4_lds(int M, int N, int K) {
  return static_cast<long>(M) * (K / 2) < (1L << 31) && static_cast<long>(N) * (K / 2) < (1L << 31);
}

}  // namespace

namespace wush {

wush_status gemm_int4_direct(int M, int N, int K, const uint8_t* A, const uint16_t* SA, const uint8_t* B,
                             const uint16_t* SB, float* Y, hipStream_t stream);

size_t gemm_int4_ws_bytes(int M, int N, int K) {
  if (M < 1 || N < 1 || K < 1 || !use_int4_lds(M, N, K)) return 0;
  const size_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN, nb = (K + 255) / 256;
  return nb * (tiles_m * kScaleA + tiles_n * kScaleB);
}

wush_status gemm_int4(int M, int N, int K, const uint8_t* A, const uint16_t* SA, const uint8_t* B,
                      const uint16_t* SB, float* Y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!use_int4_lds(M, N, K)) return gemm_int4_direct(M, N, K, A, SA, B, SB, Y, stream);
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN, nb = (K + 255) / 256;
  const long tiles = static_cast<long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffL || tiles_m + tiles_n > 65535 || nb > 65535)
    return fail(WUSH_E_SHAPE, "wush_w4a4_gemm (int4): too many tiles");
  const size_t p_bytes = gemm_int4_ws_bytes(M, N, K);
  uint8_t* P = static_cast<uint8_t*>(ws);
  if (P) {
    if (ws_bytes < p_bytes) return fail(WUSH_E_ARG, "wush_w4a4_gemm: workspace of %zu bytes, need %zu", ws_bytes, p_bytes);
  } else {
    const hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&P), p_bytes, stream);
    if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm scratch (%zu bytes): %s", p_bytes, hipGetErrorString(e));
  }
  uint8_t* PA = P;
  uint8_t* PB = P + static_cast<size_t>(nb) * tiles_m * kScaleA;
  hipLaunchKernelGGL(int4_scales_to_planes, dim3(nb, tiles_m + tiles_n), dim3(256), 0, stream, SA, M, SB, N, tiles_m,
                     K, nb, PA, PB);
  hipLaunchKernelGGL(gemm_int4_lds, dim3(static_cast<unsigned>(tiles)), dim3(512), 0, stream, A, PA, B, PB, Y, M, N, K);
  const hipError_t e = hipGetLastError();
  const hipError_t f = ws ? hipSuccess : hipFreeAsync(P, stream);
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm (int4) launch: %s", hipGetErrorString(e));
  if (f != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm scratch free: %s", hipGetErrorString(f));
  return WUSH_OK;
}

}  // namespace wush
