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

// ---------------------------------------------------------------------------
// LDS-staged kernel (any K % 128 == 0).
//
// Workgroup tile 256 x 256, four waves of 128 x 128 each (2 x 2): per K step
// of 256 a wave reads 32 fragments (32 KB) from LDS and issues 128 MFMAs, so
// LDS reads stay at 16 bytes per clock per wave.  The 256 accumulator
// registers per lane live in AGPRs; occupancy is one wave per SIMD.
//
// Global -> LDS: one K step moves 256 rows x 128 bytes of each operand.  Each
// buffer_load_dwordx4 covers 8 rows x one full 128-byte line (8 lanes per row),
// so every L2 request is a whole line; the data lands in VGPRs one step ahead
// of use and is then written to LDS with ds_write_b128.  (Measured on MI355X:
// 16-byte-per-lane LDS DMA of the same bytes keeps the texture address unit
// saturated and runs ~1.5x slower, and 64-byte row pieces halve the request
// size again.)
//
// LDS layout: a 16-row x 128-byte block per row group (both MFMA sub-steps of
// the step), 16-byte chunk c of row r stored at chunk c ^ ((r >> 1) & 7).  Both
// the writes (8 lanes per row) and the MFMA reads (16 rows, one chunk each, per
// 16-lane phase) then touch 16 distinct 4-bank groups: no bank conflicts.
// E8M0 scales (8 per row per step: 4 per MFMA sub-step) are stored as
// [rr][sub-step][16 rows][4 bytes] with a 144-byte pitch per lane row rr (another
// conflict-free spread), so a lane finds the sub-step scales of its 8 rows in
// 32 contiguous bytes.
//
// The two LDS stages are distinct __shared__ arrays and the K loop is unrolled
// by two, so every access names its array statically and the compiler knows
// that writing the next stage does not alias reading the current one.
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin (id % 8), so the
// tile index is remapped to give each XCD a contiguous run of tiles, walked in
// groups of kGroupM tile rows; the 32 CUs of an XCD then share A and B panels
// in their own L2.

constexpr int kBM = 256, kBN = 256;
constexpr int kFragStage = 2 * 16 * 2048;        // operands x row groups x (16 rows x 128 B)
constexpr int kScalePitch = 144;                 // bytes per lane row rr in the scale area
constexpr int kScaleOp = 16 * kScalePitch;       // one operand's scales for one step
constexpr int kStageBytes = kFragStage + 2 * kScaleOp;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[kStageBytes];

template <int S>
__device__ __forceinline__ uint8_t* stage_buf() {
  if constexpr (S == 0) return g_stage0;
  else return g_stage1;
}

// Buffer descriptor over `bytes` bytes at `base` (raw, unswizzled; dword 3 =
// 0x00020000 selects 32-bit data format for untyped buffer access on CDNA).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// Workgroup barrier without the release/acquire fence of __syncthreads(): that
// fence would also wait for the next stage's global loads.  LDS needs no cache
// maintenance; waiting for this wave's own LDS traffic first (lgkmcnt(0))
// orders its writes before, and its reads of a buffer before the rewrite of it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

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

struct Staging {
  uint4 a[8], b[8];   // 8 rows x 128 B per instruction, this wave's 64 rows of A and of B
  uint2 s[2];         // 64 rows x 8 scale bytes per instruction, operand (wave >> 1)
};

struct GemmCtx {
  __amdgpu_buffer_rsrc_t ra, rb, rs;
  uint32_t a_off, b_off;   // loader row r0 = 64 wave + lane / 8, chunk lane % 8
  uint32_t s_off[2];       // loader scale rows (wave & 1) 128 + 64 u + lane
  uint32_t w_frag;         // LDS byte offset of this lane's chunk within a 16-row block (instruction u even)
  uint32_t w_frag1;        // same for odd u (rows 8..15 of the block)
  uint32_t w_scale[2];     // LDS byte offset of this lane's scale row (per u)
  uint32_t r_frag[2];      // LDS byte offset of this lane's read chunk, per sub-step j
  uint32_t r_scale_a, r_scale_b;
  int wave, lane, wm, wn, nks;
  bool half_tail;              // K % 256 == 128: the last step has one MFMA sub-step
  uint32_t a_step8, b_step8;   // byte distance of 8 rows in A / B (8 * K / 2)
};

__device__ __forceinline__ void load_stage(const GemmCtx& c, int k, Staging& g) {
  const uint32_t kb = static_cast<uint32_t>(k) * 128;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    g.a[u] = load16(c.ra, c.a_off + u * c.a_step8, kb);
    g.b[u] = load16(c.rb, c.b_off + u * c.b_step8, kb);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) g.s[u] = load8(c.rs, c.s_off[u], static_cast<uint32_t>(k) * 8);
}

template <int S>
__device__ __forceinline__ void store_stage(const GemmCtx& c, const Staging& g) {
  uint8_t* st = stage_buf<S>();
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    // instruction u covers rows 64 wave + 8 u .. of the tile = row group 4 wave + u / 2
    const uint32_t blk = (4 * c.wave + u / 2) * 2048 + ((u & 1) ? c.w_frag1 : c.w_frag);
    *reinterpret_cast<uint4*>(st + blk) = g.a[u];
    *reinterpret_cast<uint4*>(st + 16 * 2048 + blk) = g.b[u];
  }
  uint8_t* ss = st + kFragStage + (c.wave >> 1) * kScaleOp;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    *reinterpret_cast<uint32_t*>(ss + c.w_scale[u]) = g.s[u].x;        // sub-step 0 scales of the row
    *reinterpret_cast<uint32_t*>(ss + c.w_scale[u] + 64) = g.s[u].y;   // sub-step 1
  }
}

// One K step (256) on stage S: read its fragments and scales, refill the other
// stage from the staging registers, start the global loads two steps ahead,
// then the 128 MFMAs.
template <int S>
__device__ __forceinline__ void k_step(const GemmCtx& c, int k, Staging& g, v4f (&acc)[8][8]) {
  stage_barrier();
  const uint8_t* st = stage_buf<S>();
  const uint32_t sh = 8u * static_cast<uint32_t>(c.lane >> 4);   // this lane's K group within the sub-step
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j == 1 && c.half_tail && k == c.nks - 1) break;   // uniform: K ends half way
    __builtin_amdgcn_sched_barrier(0);
    // 8 rows x 4 scale bytes of sub-step j for A (rows of this wave's 8 A fragments) and B
    const uint4* spa = reinterpret_cast<const uint4*>(st + kFragStage + c.r_scale_a + 64 * j);
    const uint4* spb = reinterpret_cast<const uint4*>(st + kFragStage + kScaleOp + c.r_scale_b + 64 * j);
    const uint4 a0 = spa[0], a1 = spa[1], b0 = spb[0], b1 = spb[1];
    uint4 af[8], bf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf[i] = *reinterpret_cast<const uint4*>(st + (16 + c.wn * 8 + i) * 2048 + c.r_frag[j]);
      af[i] = *reinterpret_cast<const uint4*>(st + (c.wm * 8 + i) * 2048 + c.r_frag[j]);
    }
    if (j == 0) {
      // refill the other stage from the staging registers, then start the
      // global loads two steps ahead into them.  Unconditional (clamped to the
      // last step; the surplus is never read): a conditional refill would make
      // the compiler keep two copies of the staging registers alive.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      store_stage<S ^ 1>(c, g);
      load_stage(c, min(k + 2, c.nks - 1), g);
    }
    const uint32_t sa[8] = {a0.x >> sh, a0.y >> sh, a0.z >> sh, a0.w >> sh, a1.x >> sh, a1.y >> sh, a1.z >> sh, a1.w >> sh};
    const uint32_t sb[8] = {b0.x >> sh, b0.y >> sh, b0.z >> sh, b0.w >> sh, b1.x >> sh, b1.y >> sh, b1.z >> sh, b1.w >> sh};
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][q] = mfma_fp4<0>(bf[i], sb[i], af[q], sa[q], acc[i][q]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(256, 1) void gemm_mxfp4_lds(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                        const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                        float* __restrict__ Y, int M, int N, int K) {
  GemmCtx c;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.wm = c.wave >> 1;
  c.wn = c.wave & 1;
  c.nks = (K + 255) / 256;
  c.half_tail = (K & 255) != 0;
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int rr = c.lane & 15, grp = c.lane >> 4;
  // 32-bit byte offsets from uniform bases (the host checks every operand is
  // below 2^31 bytes).  Rows past the edge read the last row (never stored).
  // A K of 128 (mod 256) leaves a half step: its upper 64 bytes per row (and 4
  // scale bytes) read past the row, the next row or zeros from the bounded
  // descriptor, and feed only the sub-step that the last step skips.
  const uint32_t krow = static_cast<uint32_t>(K) / 2, srow = static_cast<uint32_t>(K) / 32;
  const int lr = c.lane >> 3, lc = c.lane & 7;
  const int ra = min(m0 + 64 * c.wave + lr, M - 1), rb = min(n0 + 64 * c.wave + lr, N - 1);
  c.a_off = static_cast<uint32_t>(ra) * krow + lc * 16;
  c.b_off = static_cast<uint32_t>(rb) * krow + lc * 16;
  c.a_step8 = 8 * krow;
  c.b_step8 = 8 * krow;
  const int s_op = c.wave >> 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = (c.wave & 1) * 128 + 64 * u + c.lane;            // row within the tile
    const int base = s_op ? n0 : m0, lim = s_op ? N - 1 : M - 1;
    c.s_off[u] = static_cast<uint32_t>(min(base + row, lim)) * srow;
    // scale position: lane row rr' = row % 16, then [sub-step][half = row / 128][i = (row / 16) % 8]
    c.w_scale[u] = (row & 15) * kScalePitch + ((row >> 7) * 8 + ((row >> 4) & 7)) * 4;
  }
  // writer chunk position: row r = lr (+8 for odd u), logical chunk lc
  c.w_frag = lr * 128 + ((lc ^ ((lr >> 1) & 7)) * 16);
  c.w_frag1 = (lr + 8) * 128 + ((lc ^ (((lr + 8) >> 1) & 7)) * 16);
  // reader: row rr, logical chunk 4 j + grp
#pragma unroll
  for (int j = 0; j < 2; ++j) c.r_frag[j] = rr * 128 + ((((4 * j + grp) ^ ((rr >> 1) & 7))) * 16);
  c.r_scale_a = rr * kScalePitch + c.wm * 32;
  c.r_scale_b = rr * kScalePitch + c.wn * 32;
  // descriptors bound the operands exactly (out-of-range lanes read zeros)
  c.ra = make_rsrc(A, static_cast<uint32_t>(M) * krow);
  c.rb = make_rsrc(B, static_cast<uint32_t>(N) * krow);
  c.rs = s_op ? make_rsrc(SB, static_cast<uint32_t>(N) * srow) : make_rsrc(SA, static_cast<uint32_t>(M) * srow);

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};

  Staging g;
  load_stage(c, 0, g);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  store_stage<0>(c, g);
  load_stage(c, min(1, c.nks - 1), g);
  int k = 0;
#pragma unroll 1
  for (; k + 1 < c.nks; k += 2) {
    k_step<0>(c, k, g, acc);
    k_step<1>(c, k + 1, g, acc);
  }
  if (k < c.nks) k_step<0>(c, k, g, acc);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // surplus staging loads

  // lane holds Y[m0 + 128 wm + 16 q + rr][n0 + 128 wn + 16 i + 4 grp + 0..3]
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int m = m0 + c.wm * 128 + q * 16 + rr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + c.wn * 128 + i * 16 + 4 * grp;
      float* dst = Y + static_cast<size_t>(m) * N + n;
      if (n + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[i][q][0], acc[i][q][1], acc[i][q][2], acc[i][q][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) dst[e] = acc[i][q][e];
      }
    }
  }
}

}  // namespace

namespace wush {

wush_status gemm_mxfp4(int M, int N, int K, const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                       float* Y, hipStream_t stream) {
  const bool small = static_cast<long>(M) * (K / 2) < (1L << 31) && static_cast<long>(N) * (K / 2) < (1L << 31);
  if (small) {
    const long tiles = static_cast<long>((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    if (tiles > 0x7fffffffL) return fail(WUSH_E_SHAPE, "wush_w4a4_gemm: too many tiles");
    hipLaunchKernelGGL(gemm_mxfp4_lds, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, A, SA, B, SB, Y, M,
                       N, K);
  } else {
    dim3 grid((N + kBlockN - 1) / kBlockN, (M + kBlockM - 1) / kBlockM);
    if (grid.y > 65535u) return fail(WUSH_E_SHAPE, "wush_w4a4_gemm: M=%d too large", M);
    hipLaunchKernelGGL(gemm_mxfp4_direct, grid, dim3(256), 0, stream, A, SA, B, SB, Y, M, N, K);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // namespace wush
