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
// LDS-staged kernel (K % 256 == 0).
//
// Workgroup tile 256 x 256, four waves of 128 x 128 each (2 x 2), so every
// wave issues 64 MFMAs per 16 fragment reads from LDS: 16 bytes per clock per
// wave, well inside the LDS bandwidth.  The 256 accumulator registers per
// lane live in AGPRs; occupancy is one wave per SIMD.
//
// Staging: one K step of 256 moves 256 rows x 128 bytes of each operand.
// Each 1 KB fragment (16 rows x 128 K values of one MFMA sub-step) is brought
// from global memory straight into LDS with global_load_lds_dwordx4, lane l
// landing at byte 16 l of the fragment, which is exactly where the consuming
// MFMA lane l reads it back with one ds_read_b128: both sides are
// lane-linear, so there are no bank conflicts.  Two stages (128 KB) are
// double-buffered; stage ks+1 is loaded while stage ks feeds the MFMAs.
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin (id % 8), so the
// tile index is remapped to give each XCD a contiguous run of tiles, walked in
// groups of kGroupM tile rows; the 32 CUs of an XCD then share A and B panels
// in their own L2.

constexpr int kBM = 256, kBN = 256;
constexpr int kFragBytes = 2 * 16 * 2 * 1024;    // operands x row groups x sub-steps x fragment
constexpr int kScaleBytes = 2 * 256 * 8;          // operands x rows x 8 scale bytes of one K step
constexpr int kStageBytes = kFragBytes + kScaleBytes;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer descriptor over `bytes` bytes at `base` (raw, unswizzled; dword 3 =
// 0x00020000 selects 32-bit data format for untyped buffer access on CDNA).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// 16 bytes per lane from (voffset + soffset) straight into LDS at
// lds_frag + 16 * lane (buffer_load_dwordx4 ... lds; M0 holds the LDS base).
// The instruction's immediate offset would move the LDS destination as well,
// so any uniform displacement goes into soffset instead.
__device__ __forceinline__ void load_frag_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_frag) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds_frag), 16, voff, soff, 0, 0);
}

// 4 bytes per lane into LDS at lds_dst + 4 * lane.
__device__ __forceinline__ void load_dword_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds_dst), 4, voff, soff, 0, 0);
}

__device__ __forceinline__ uint4 read_frag(const uint8_t* lds_frag, int lane) {
  return *reinterpret_cast<const uint4*>(lds_frag + lane * 16);
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

__global__ __launch_bounds__(256, 1) void gemm_mxfp4_lds(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                                        const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                        float* __restrict__ Y, int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int rr = lane & 15, grp = lane >> 4;

  // 32-bit per-lane byte offsets from the uniform base pointers (the host checks
  // that every operand is below 2^31 bytes), so loads use scalar-base addressing.
  // loader: this wave stages row groups 4*wave .. 4*wave+3 of both operands
  const uint32_t krow = static_cast<uint32_t>(K) / 2, srow = static_cast<uint32_t>(K) / 32;
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int ra = min(m0 + (4 * wave + t) * 16 + rr, M - 1);
    const int rb = min(n0 + (4 * wave + t) * 16 + rr, N - 1);
    a_off[t] = static_cast<uint32_t>(ra) * krow + grp * 32;
    b_off[t] = static_cast<uint32_t>(rb) * krow + grp * 32;
  }
  // scales: this wave stages 128 rows (half (wave & 1)) of one operand's 8 scale
  // bytes per K step; one LDS DMA moves 64 lanes x 4 bytes = 32 rows, lane l
  // fetching half (l % 2) of row 32 c + l / 2, so four instructions per wave
  const int s_op = wave >> 1;                         // 0: A scales, 1: B scales
  uint32_t s_off[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = (wave & 1) * 128 + c * 32 + (lane >> 1);
    const int lim = s_op ? N - 1 : M - 1;
    const int base = s_op ? n0 : m0;
    s_off[c] = static_cast<uint32_t>(min(base + row, lim)) * srow + (lane & 1) * 4;
  }
  // consumer: wave (wm, wn) owns rows m0 + 128 wm .., cols n0 + 128 wn ..
  const int wm = wave >> 1, wn = wave & 1;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, static_cast<uint32_t>(M) * krow);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, static_cast<uint32_t>(N) * krow);
  const __amdgpu_buffer_rsrc_t rs = s_op ? make_rsrc(SB, static_cast<uint32_t>(N) * srow)
                                         : make_rsrc(SA, static_cast<uint32_t>(M) * srow);

  auto issue_stage = [&](int ks, int buf) {
    uint8_t* st = smem + buf * kStageBytes;
    const uint32_t kb = static_cast<uint32_t>(ks) * 128;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rg = 4 * wave + t;
      load_frag_lds(ra, a_off[t], kb, st + ((0 * 16 + rg) * 2 + 0) * 1024);
      load_frag_lds(ra, a_off[t], kb + 16, st + ((0 * 16 + rg) * 2 + 1) * 1024);
      load_frag_lds(rb, b_off[t], kb, st + ((1 * 16 + rg) * 2 + 0) * 1024);
      load_frag_lds(rb, b_off[t], kb + 16, st + ((1 * 16 + rg) * 2 + 1) * 1024);
    }
    // scale rows [row][8 bytes], A then B
    uint8_t* ss = st + kFragBytes + s_op * 2048 + (wave & 1) * 1024;
#pragma unroll
    for (int c = 0; c < 4; ++c) load_dword_lds(rs, s_off[c], static_cast<uint32_t>(ks) * 8, ss + c * 256);
  };

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nks = K / 256;
  issue_stage(0, 0);
#pragma unroll 1
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // everything this step needs goes from LDS into registers before the next
    // stage's LDS DMA is issued: an LDS read issued after an LDS DMA must wait
    // for it (the compiler cannot tell the two stage buffers apart)
    const uint8_t* st = smem + buf * kStageBytes;
    uint4 af[2][8], bf[2][8];
    uint32_t sa[8], sb[8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        af[j][i] = read_frag(st + ((0 * 16 + wm * 8 + i) * 2 + j) * 1024, lane);
        bf[j][i] = read_frag(st + ((1 * 16 + wn * 8 + i) * 2 + j) * 1024, lane);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sa[i] = *reinterpret_cast<const uint16_t*>(st + kFragBytes + (wm * 128 + i * 16 + rr) * 8 + grp * 2);
      sb[i] = *reinterpret_cast<const uint16_t*>(st + kFragBytes + 2048 + (wn * 128 + i * 16 + rr) * 8 + grp * 2);
    }
    if (ks + 1 < nks) issue_stage(ks + 1, buf ^ 1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = mfma_fp4<0>(bf[0][i], sb[i], af[0][q], sa[q], acc[i][q]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = mfma_fp4<1>(bf[1][i], sb[i], af[1][q], sa[q], acc[i][q]);
  }

  // lane holds Y[m0 + 128 wm + 16 q + rr][n0 + 128 wn + 16 i + 4 grp + 0..3]
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int m = m0 + wm * 128 + q * 16 + rr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wn * 128 + i * 16 + 4 * grp;
      float* dst = Y + static_cast<size_t>(m) * N + n;
      if (n + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[i][q][0], acc[i][q][1], acc[i][q][2], acc[i][q][3]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (n + c < N) dst[c] = acc[i][q][c];
      }
    }
  }
}

}  // namespace

namespace wush {

wush_status gemm_mxfp4(int M, int N, int K, const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                       float* Y, hipStream_t stream) {
  if (K % 256 == 0) {
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
