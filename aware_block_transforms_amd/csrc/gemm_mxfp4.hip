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

#include <algorithm>
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
// LDS-staged, software-pipelined kernel (K >= 256, K % 128 == 0).
//
// Workgroup tile 256 x 256, four waves of 128 x 128 each (2 x 2); the 256
// accumulator registers per lane live in AGPRs (one wave per SIMD).  K is
// staged through LDS in blocks of 256 and consumed in sub-steps of 128: per
// sub-step ("phase") a wave issues 64 MFMAs and reads 16 fragments (16 KB).
//
// Pipeline, per phase p = 2 k + j (block k, sub-step j), overlapped with the
// MFMAs of p, which take their operands from registers:
//   * LDS reads of sub-step p+1 into the other fragment register set (the A
//     fragments one by one, each right after the MFMAs that free its
//     registers),
//   * j = 0: LDS writes of block k+1's B operand from its staging registers,
//     then the global loads of block k+2's B into them;
//     j = 1: the same for A, blocks k+2 and k+3,
// and after the j = 0 phase one workgroup barrier (one per block suffices: a
// j = 1 phase reads block k+1 and writes block k's buffer, whose last reads
// came before the barrier; the next barrier publishes both writes before any
// wave reads them).  Two LDS block buffers (68 KB each); every global load has
// two phases to land.
//
// Global -> registers: buffer_load_dwordx4 with lane (lr, lc) = (lane / 8,
// lane % 8) fetching the 16-byte chunk lc of row lr: 8 full 128-byte rows
// (one block of one row) per instruction.
// LDS layout of a 2 KB fragment pair (16 rows x 128 B, both sub-steps): chunk
// c of row r at 16-byte slot 8 r + (c ^ ((r >> 1) & 7)); a ds_write_b128
// (16 lanes: two rows) and a ds_read_b128 (16 lanes: rows 0..15 of one chunk)
// both touch all 64 banks once.
// E8M0 scales, one byte each, as plane [sub-step j][K group g] of
// [lane row rr][8 half + i] for tile row 128 half + 16 i + rr: a lane reads
// the 8 scale bytes of its 8 fragments with one ds_read_b64 and the MFMA's
// op_sel picks the byte; planes of odd K groups are rotated by 8 bytes so
// that the lane groups of K groups 2m and 2m+1 read disjoint banks.  A small
// pre-pass writes the scales in exactly this order, 2 KB per (row tile,
// block), so that staging them is one contiguous 8-byte load and one
// ds_write_b64 per lane (row-major scales would cost a cache line per row).
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin (id % 8), so the
// tile index is remapped to give each XCD a contiguous run of tiles, walked in
// groups of kGroupM tile rows; the 32 CUs of an XCD then share A and B panels
// in their own L2.

constexpr int kBM = 256, kBN = 256;
constexpr int kFragOp = 16 * 2048;                 // one operand of one block: 16 fragment pairs
constexpr int kScaleOp = 8 * 256;                  // one operand's scale planes
constexpr int kStageBytes = 2 * kFragOp + 2 * kScaleOp;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw, unswizzled; dword 3 = 0x00020000 selects 32-bit data format for untyped access on CDNA
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// s_waitcnt immediates (gfx9 layout: vmcnt [3:0] + [15:14], expcnt [6:4],
// lgkmcnt [11:8]); issued through the builtin so that the compiler's own wait
// insertion knows which loads have completed.
constexpr unsigned kWaitLgkm0 = 0xC07F;   // lgkmcnt(0)
constexpr unsigned kWaitVm0 = 0x0F70;     // vmcnt(0)

// All of this wave's LDS traffic done, then the workgroup barrier.  No memory
// fence (that of __syncthreads() would also wait for the in-flight global
// loads): only LDS is shared, and lgkmcnt(0) orders this wave's writes before,
// and its reads of a buffer before any rewrite of it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

struct Frags { uint4 a[8], b[8]; uint2 sa, sb; };   // sa / sb: 8 scale bytes, fragment i in byte i
// one operand of one block: this wave's 64 rows of codes and its quarter
// (512 bytes) of the block's scale planes
struct Stage { uint4 d[8]; uint2 s; };

struct GemmCtx {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  uint32_t a_off, b_off;         // loader: row 64 wave + lane / 8, chunk lane % 8 (+ u * row_step8 for instruction u)
  uint32_t row_step8;            // bytes of 8 rows
  uint32_t sa_off, sb_off;       // this lane's 8 bytes of the tile's plane-ordered scales, block 0
  uint32_t w_frag0, w_frag1;     // LDS slot of the loader's chunk within a fragment pair (even / odd u)
  uint32_t w_scale;              // LDS offset of the loader's 8 scale bytes within the operand's planes
  uint32_t r_frag[2];            // LDS slot of this lane's read chunk within a fragment pair, per sub-step
  uint32_t r_scale_a, r_scale_b; // LDS offset of this lane's 8 scale bytes within plane (0, g)
  int wave, wm, wn, nb;
};

__device__ __forceinline__ void load_op(__amdgpu_buffer_rsrc_t rd, uint32_t d_off, __amdgpu_buffer_rsrc_t rs,
                                        uint32_t s_off, uint32_t step8, int k, Stage& g, uint32_t dbase = 0,
                                        uint32_t sbase = 0) {
#pragma unroll
  for (int u = 0; u < 8; ++u) g.d[u] = load16(rd, d_off, dbase + static_cast<uint32_t>(k) * 128 + u * step8);
  g.s = load8(rs, s_off, sbase + static_cast<uint32_t>(k) * kScaleOp);
}

// one operand (op 0 = A, 1 = B) of a block into the LDS buffer `buf`
__device__ __forceinline__ void write_op(const GemmCtx& c, uint8_t* buf, int op, const Stage& g) {
  uint8_t* fb = buf + op * kFragOp + c.wave * (4 * 2048);
#pragma unroll
  for (int u = 0; u < 8; ++u)
    *reinterpret_cast<uint4*>(fb + (u >> 1) * 2048 + ((u & 1) ? c.w_frag1 : c.w_frag0)) = g.d[u];
  *reinterpret_cast<uint2*>(buf + 2 * kFragOp + op * kScaleOp + c.w_scale) = g.s;
}

__device__ __forceinline__ uint4 read_a(const GemmCtx& c, const uint8_t* buf, int j, int q) {
  return *reinterpret_cast<const uint4*>(buf + (c.wm * 8 + q) * 2048 + c.r_frag[j]);
}

// B fragments and both operands' scales of sub-step j of the block in `buf`
__device__ __forceinline__ void read_b_scales(const GemmCtx& c, const uint8_t* buf, int j, Frags& f) {
  f.sa = *reinterpret_cast<const uint2*>(buf + 2 * kFragOp + j * 1024 + c.r_scale_a);
  f.sb = *reinterpret_cast<const uint2*>(buf + 2 * kFragOp + kScaleOp + j * 1024 + c.r_scale_b);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    f.b[i] = *reinterpret_cast<const uint4*>(buf + kFragOp + (c.wn * 8 + i) * 2048 + c.r_frag[j]);
}

// MFMA for B fragment I and A fragment Q: scale bytes I and Q sit in byte I % 4
// (resp. Q % 4) of dword I / 4 (Q / 4).
template <int I, int Q>
__device__ __forceinline__ void mfma_iq(const Frags& f, v4f& acc) {
  const uint32_t sb = (I < 4) ? f.sb.x : f.sb.y;
  const uint32_t sa = (Q < 4) ? f.sa.x : f.sa.y;
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_operand(f.b[I]), as_operand(f.a[Q]), acc, 4, 4, I % 4,
                                                         static_cast<int>(sb), Q % 4, static_cast<int>(sa));
}

template <int Q>
__device__ __forceinline__ void mfma_column(const Frags& f, v4f (&acc)[8][8]) {
  mfma_iq<0, Q>(f, acc[0][Q]);
  mfma_iq<1, Q>(f, acc[1][Q]);
  mfma_iq<2, Q>(f, acc[2][Q]);
  mfma_iq<3, Q>(f, acc[3][Q]);
  mfma_iq<4, Q>(f, acc[4][Q]);
  mfma_iq<5, Q>(f, acc[5][Q]);
  mfma_iq<6, Q>(f, acc[6][Q]);
  mfma_iq<7, Q>(f, acc[7][Q]);
}

// Slot Q of a phase: the 8 MFMAs of column Q of the current sub-step on
// `cur`, interleaved with this slot's share of the memory work so that no
// unit sees a burst: B fragments 2Q and 2Q+1 of the next sub-step into `nxt`
// (slots 0-3, so that they have landed when the next phase starts), staging
// register Q written to LDS and reloaded from the next block of its operand,
// scale plane Q written, and at the end A fragment Q of the next sub-step
// into the registers that column Q just released.  The scheduling fences
// keep this order: the compiler would otherwise hoist all LDS reads and hold
// both fragment sets at once.
template <int Q>
__device__ __forceinline__ void slot(const GemmCtx& c, const uint8_t* rbuf, int rj, uint8_t* fb, uint2* sp,
                                     __amdgpu_buffer_rsrc_t rd, uint32_t d_off, __amdgpu_buffer_rsrc_t rs,
                                     uint32_t s_off, uint32_t dso, uint32_t sso, const Frags& cur, Frags& nxt,
                                     Stage& st, v4f (&acc)[8][8]) {
  mfma_iq<0, Q>(cur, acc[0][Q]);
  if constexpr (Q < 4)
    nxt.b[2 * Q] = *reinterpret_cast<const uint4*>(rbuf + kFragOp + (c.wn * 8 + 2 * Q) * 2048 + c.r_frag[rj]);
  mfma_iq<1, Q>(cur, acc[1][Q]);
  if constexpr (Q < 4)
    nxt.b[2 * Q + 1] = *reinterpret_cast<const uint4*>(rbuf + kFragOp + (c.wn * 8 + 2 * Q + 1) * 2048 + c.r_frag[rj]);
  *reinterpret_cast<uint4*>(fb + (Q >> 1) * 2048 + ((Q & 1) ? c.w_frag1 : c.w_frag0)) = st.d[Q];
  mfma_iq<2, Q>(cur, acc[2][Q]);
  st.d[Q] = load16(rd, d_off, dso + Q * c.row_step8);
  mfma_iq<3, Q>(cur, acc[3][Q]);
  if (Q == 6) *sp = st.s;
  mfma_iq<4, Q>(cur, acc[4][Q]);
  if (Q == 7) st.s = load8(rs, s_off, sso);
  mfma_iq<5, Q>(cur, acc[5][Q]);
  mfma_iq<6, Q>(cur, acc[6][Q]);
  mfma_iq<7, Q>(cur, acc[7][Q]);
  nxt.a[Q] = read_a(c, rbuf, rj, Q);
  __builtin_amdgcn_sched_barrier(0);
}

// One phase: the MFMAs of the current sub-step on `cur`; meanwhile sub-step
// (rbuf, rj) into `nxt`, operand `op` of the block staged in `st` written to
// `wbuf`, and `st` reloaded from the block at byte offsets dso (codes) and
// sso (scale planes) past the lane's own offsets.
template <bool kBarrier>
__device__ __forceinline__ void phase(const GemmCtx& c, const uint8_t* rbuf, int rj, uint8_t* wbuf, int op,
                                      uint32_t dso, uint32_t sso, Frags& cur, Frags& nxt, Stage& st,
                                      v4f (&acc)[8][8]) {
  __builtin_amdgcn_sched_barrier(0);
  nxt.sa = *reinterpret_cast<const uint2*>(rbuf + 2 * kFragOp + rj * 1024 + c.r_scale_a);
  nxt.sb = *reinterpret_cast<const uint2*>(rbuf + 2 * kFragOp + kScaleOp + rj * 1024 + c.r_scale_b);
  uint8_t* const fb = wbuf + op * kFragOp + c.wave * (4 * 2048);
  uint2* const sp = reinterpret_cast<uint2*>(wbuf + 2 * kFragOp + op * kScaleOp + c.w_scale);
  const __amdgpu_buffer_rsrc_t rd = op ? c.rb : c.ra, rs = op ? c.rsb : c.rsa;
  const uint32_t d_off = op ? c.b_off : c.a_off, s_off = op ? c.sb_off : c.sa_off;
  slot<0>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  slot<1>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  slot<2>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  slot<3>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  slot<4>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  slot<5>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  slot<6>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  slot<7>(c, rbuf, rj, fb, sp, rd, d_off, rs, s_off, dso, sso, cur, nxt, st, acc);
  if (kBarrier) phase_barrier();
}

// Scales in plane order: for each 256-row tile t and 256-wide K block k, the
// 2 KB at (t nb + k) * 2048 hold the block's 8 planes exactly as the LDS
// stage stores them (see above); rows past the operand and K groups past K
// are zero.  One workgroup of 256 threads (thread = tile row) per row tile
// and pair of blocks.  Tiles 0 .. tiles_a - 1 come from SA (ra rows), the
// rest from SB (rb rows).
__global__ __launch_bounds__(256) void scales_to_planes(const uint8_t* __restrict__ SA, int ra,
                                                        const uint8_t* __restrict__ SB, int rb, int tiles_a, int K,
                                                        int nb, uint8_t* __restrict__ P) {
  __shared__ uint8_t planes[2 * kScaleOp];
  const int t = blockIdx.x, k0 = 2 * blockIdx.y, tr = threadIdx.x;
  const bool in_a = t < tiles_a;
  const int row = (in_a ? t : t - tiles_a) * kBM + tr;
  const int rows = in_a ? ra : rb;
  const int sdw = K / 128;   // scale dwords per row
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(in_a ? SA : SB) + static_cast<size_t>(row) * sdw;
  uint32_t v[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) v[d] = (row < rows && 2 * k0 + d < sdw) ? s32[2 * k0 + d] : 0u;
  const int rr = tr & 15, pos = 8 * (tr >> 7) + ((tr >> 4) & 7);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int b = 0; b < 8; ++b)
      planes[kk * kScaleOp + b * 256 + rr * 16 + (pos ^ (8 * (b & 1)))] =
          static_cast<uint8_t>(v[2 * kk + (b >> 2)] >> (8 * (b & 3)));
  __syncthreads();
  const int nk = min(2, nb - k0);   // 16 bytes per thread per block pair
  if (tr * 16 < nk * kScaleOp)
    *reinterpret_cast<uint4*>(P + (static_cast<size_t>(t) * nb + k0) * kScaleOp + tr * 16) =
        reinterpret_cast<const uint4*>(planes)[tr];
}

__global__ __launch_bounds__(256, 1) void gemm_mxfp4_lds(const uint8_t* __restrict__ A, const uint8_t* __restrict__ PA,
                                                        const uint8_t* __restrict__ B, const uint8_t* __restrict__ PB,
                                                        float* __restrict__ Y, int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];
  GemmCtx c;
  const int lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.wm = c.wave >> 1;
  c.wn = c.wave & 1;
  const int nfull = K / 256;                 // >= 1 (checked by the launcher)
  const bool half = (K & 255) != 0;          // a last block of one sub-step
  c.nb = nfull + (half ? 1 : 0);
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int rr = lane & 15, grp = lane >> 4;
  // 32-bit byte offsets from uniform bases (the host checks every operand is
  // below 2^31 bytes).  Rows past the edge fall outside the buffer descriptor's
  // bound and read as zeros (their outputs are never stored).  In a half block
  // the upper 64 bytes of a row read the next row's data or zeros; they feed
  // only the sub-step that is skipped.
  const uint32_t krow = static_cast<uint32_t>(K) / 2;
  const int lr = lane >> 3, lc = lane & 7;
  c.a_off = static_cast<uint32_t>(m0 + 64 * c.wave + lr) * krow + lc * 16;
  c.b_off = static_cast<uint32_t>(n0 + 64 * c.wave + lr) * krow + lc * 16;
  c.row_step8 = 8 * krow;
  c.w_frag0 = lr * 128 + ((lc ^ ((lr >> 1) & 7)) * 16);
  c.w_frag1 = (lr + 8) * 128 + ((lc ^ (((lr + 8) >> 1) & 7)) * 16);
  {
    // scales arrive already in plane order, one 2 KB block per (row tile,
    // K block): wave w copies bytes 512 w + 8 lane .. + 7
    c.w_scale = c.wave * 512 + lane * 8;
    c.sa_off = static_cast<uint32_t>(tm * c.nb) * kScaleOp + c.w_scale;
    c.sb_off = static_cast<uint32_t>(tn * c.nb) * kScaleOp + c.w_scale;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) c.r_frag[j] = rr * 128 + ((((4 * j + grp) ^ ((rr >> 1) & 7))) * 16);
  // odd K groups keep their planes rotated by 8 bytes, so that the two lane
  // groups of a ds_read_b64 half (K groups 2m and 2m+1) use disjoint banks
  c.r_scale_a = grp * 256 + rr * 16 + ((c.wm * 8) ^ (8 * (grp & 1)));
  c.r_scale_b = grp * 256 + rr * 16 + ((c.wn * 8) ^ (8 * (grp & 1)));
  c.ra = make_rsrc(A, static_cast<uint32_t>(M) * krow);
  c.rb = make_rsrc(B, static_cast<uint32_t>(N) * krow);
  c.rsa = make_rsrc(PA, static_cast<uint32_t>(tiles_m * c.nb) * kScaleOp);
  c.rsb = make_rsrc(PB, static_cast<uint32_t>(tiles_n * c.nb) * kScaleOp);

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};

  uint8_t* const buf0 = smem;
  uint8_t* const buf1 = smem + kStageBytes;
  const int last = c.nb - 1;
  // prologue: block 0 and block 1's A into LDS, block 1's B and block 2's A
  // into the staging registers, sub-step (0, 0) into the first fragment set.
  // Fenced so that the staging loads keep the order the main loop assumes
  // (B before A).
  Stage sa, sb;
  Frags f0, f1;
  load_op(c.ra, c.a_off, c.rsa, c.sa_off, c.row_step8, 0, sa);
  load_op(c.rb, c.b_off, c.rsb, c.sb_off, c.row_step8, 0, sb);
  __builtin_amdgcn_sched_barrier(0);
  write_op(c, buf0, 0, sa);
  write_op(c, buf0, 1, sb);
  __builtin_amdgcn_sched_barrier(0);
  load_op(c.ra, c.a_off, c.rsa, c.sa_off, c.row_step8, min(1, last), sa);
  __builtin_amdgcn_sched_barrier(0);
  load_op(c.rb, c.b_off, c.rsb, c.sb_off, c.row_step8, min(1, last), sb);
  __builtin_amdgcn_sched_barrier(0);
  write_op(c, buf1, 0, sa);
  __builtin_amdgcn_sched_barrier(0);
  load_op(c.ra, c.a_off, c.rsa, c.sa_off, c.row_step8, min(2, last), sa);
  phase_barrier();
  read_b_scales(c, buf0, 0, f0);
#pragma unroll
  for (int q = 0; q < 8; ++q) f0.a[q] = read_a(c, buf0, 0, q);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_sched_barrier(0);

  // The loop runs at least once, so every path consumes the prologue's staging
  // loads and the compiler cannot sink (and reorder) them past the loop entry.
  int k = 0;
#pragma unroll 1
  do {
    uint8_t* const cb = (k & 1) ? buf1 : buf0;   // block k
    uint8_t* const nb = (k & 1) ? buf0 : buf1;   // block k + 1
    // sub-step (k, 0); read (k, 1); write B(k+1); load B(k+2); barrier
    const uint32_t kb = static_cast<uint32_t>(min(k + 2, last)), ka = static_cast<uint32_t>(min(k + 3, last));
    phase<true>(c, cb, 1, nb, 1, kb * 128, kb * kScaleOp, f0, f1, sb, acc);
    // sub-step (k, 1); read (k+1, 0); write A(k+2) into block k's buffer; load A(k+3).
    // No barrier: block k's buffer was last read before the barrier above,
    // and A(k+2) is next read after the barrier that ends the next phase.
    phase<false>(c, nb, 0, cb, 0, ka * 128, ka * kScaleOp, f1, f0, sa, acc);
    ++k;
  } while (k < nfull);
  if (half) {   // sub-step (nfull, 0), read by the last phase
    mfma_column<0>(f0, acc); mfma_column<1>(f0, acc); mfma_column<2>(f0, acc); mfma_column<3>(f0, acc);
    mfma_column<4>(f0, acc); mfma_column<5>(f0, acc); mfma_column<6>(f0, acc); mfma_column<7>(f0, acc);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // surplus staging loads

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

// ---------------------------------------------------------------------------
// Persistent form of the LDS kernel (K a multiple of 256, at least 4 blocks):
// one workgroup per CU walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...
// (the same XCD-aware order, and the same XCD, since a workgroup id keeps its
// residue mod 8), and the software pipeline runs on across tile boundaries:
// the loads that would fall past a tile's last K block fetch the next tile's
// first blocks instead, so the next tile's first LDS block and fragments are
// ready when its MFMAs start.  Between tiles the wave only stores its output
// tile and clears its accumulators.  Buffer parity follows the global block
// count.  Offsets: a loader lane's own part (row within the tile, chunk) is in
// its voffset, the tile and block part in the scalar soffset.
struct TileBase {
  uint32_t a, b;      // code bytes of the tile's first A / B row
  uint32_t sa, sb;    // plane-ordered scale bytes of the tile's row tiles, block 0
  int m0, n0;
};

__device__ __forceinline__ TileBase tile_base(int id, int tiles_m, int tiles_n, int nb, uint32_t krow) {
  int tm, tn;
  tile_of(id, tiles_m, tiles_n, tm, tn);
  TileBase t;
  t.m0 = tm * kBM;
  t.n0 = tn * kBN;
  t.a = static_cast<uint32_t>(t.m0) * krow;
  t.b = static_cast<uint32_t>(t.n0) * krow;
  t.sa = static_cast<uint32_t>(tm * nb) * kScaleOp;
  t.sb = static_cast<uint32_t>(tn * nb) * kScaleOp;
  return t;
}

__global__ __launch_bounds__(256, 1) void gemm_mxfp4_persist(const uint8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ PA,
                                                            const uint8_t* __restrict__ B,
                                                            const uint8_t* __restrict__ PB, float* __restrict__ Y,
                                                            int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];
  GemmCtx c;
  const int lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.wm = c.wave >> 1;
  c.wn = c.wave & 1;
  c.nb = K / 256;                             // >= 4 (checked by the launcher)
  const int nb = c.nb;
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  const int ntiles = tiles_m * tiles_n;
  const int step = gridDim.x;
  int t = blockIdx.x;
  if (t >= ntiles) return;                    // workgroup-uniform
  const int rr = lane & 15, grp = lane >> 4;
  const uint32_t krow = static_cast<uint32_t>(K) / 2;
  const int lr = lane >> 3, lc = lane & 7;
  c.a_off = static_cast<uint32_t>(64 * c.wave + lr) * krow + lc * 16;
  c.b_off = c.a_off;
  c.row_step8 = 8 * krow;
  c.w_frag0 = lr * 128 + ((lc ^ ((lr >> 1) & 7)) * 16);
  c.w_frag1 = (lr + 8) * 128 + ((lc ^ (((lr + 8) >> 1) & 7)) * 16);
  c.w_scale = c.wave * 512 + lane * 8;
  c.sa_off = c.w_scale;
  c.sb_off = c.w_scale;
#pragma unroll
  for (int j = 0; j < 2; ++j) c.r_frag[j] = rr * 128 + ((((4 * j + grp) ^ ((rr >> 1) & 7))) * 16);
  c.r_scale_a = grp * 256 + rr * 16 + ((c.wm * 8) ^ (8 * (grp & 1)));
  c.r_scale_b = grp * 256 + rr * 16 + ((c.wn * 8) ^ (8 * (grp & 1)));
  c.ra = make_rsrc(A, static_cast<uint32_t>(M) * krow);
  c.rb = make_rsrc(B, static_cast<uint32_t>(N) * krow);
  c.rsa = make_rsrc(PA, static_cast<uint32_t>(tiles_m * nb) * kScaleOp);
  c.rsb = make_rsrc(PB, static_cast<uint32_t>(tiles_n * nb) * kScaleOp);

  TileBase cur = tile_base(t, tiles_m, tiles_n, nb, krow);
  TileBase nxt = tile_base(t + step < ntiles ? t + step : t, tiles_m, tiles_n, nb, krow);

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};

  uint8_t* const buf0 = smem;
  uint8_t* const buf1 = smem + kStageBytes;
  // prologue of the first tile, as in the per-tile kernel
  Stage sa, sb;
  Frags f0, f1;
  load_op(c.ra, c.a_off, c.rsa, c.sa_off, c.row_step8, 0, sa, cur.a, cur.sa);
  load_op(c.rb, c.b_off, c.rsb, c.sb_off, c.row_step8, 0, sb, cur.b, cur.sb);
  __builtin_amdgcn_sched_barrier(0);
  write_op(c, buf0, 0, sa);
  write_op(c, buf0, 1, sb);
  __builtin_amdgcn_sched_barrier(0);
  load_op(c.ra, c.a_off, c.rsa, c.sa_off, c.row_step8, 1, sa, cur.a, cur.sa);
  __builtin_amdgcn_sched_barrier(0);
  load_op(c.rb, c.b_off, c.rsb, c.sb_off, c.row_step8, 1, sb, cur.b, cur.sb);
  __builtin_amdgcn_sched_barrier(0);
  write_op(c, buf1, 0, sa);
  __builtin_amdgcn_sched_barrier(0);
  load_op(c.ra, c.a_off, c.rsa, c.sa_off, c.row_step8, 2, sa, cur.a, cur.sa);
  phase_barrier();
  read_b_scales(c, buf0, 0, f0);
#pragma unroll
  for (int q = 0; q < 8; ++q) f0.a[q] = read_a(c, buf0, 0, q);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_sched_barrier(0);

  int par = 0;                                // LDS buffer of the current block
  // Staging offsets (codes, scale planes) of the blocks iteration k reloads:
  // block k + 2 of B and k + 3 of A, of this tile or, past its end, of the
  // next one.  Kept as running offsets, one add and one select each per
  // iteration: they continue across a tile switch, since the next tile's
  // block j follows its block j - 1 at +128 bytes whichever tile loaded it.
  uint32_t dso_b = cur.b + 2 * 128u, sso_b = cur.sb + 2 * kScaleOp;
  uint32_t dso_a = cur.a + 3 * 128u, sso_a = cur.sa + 3 * kScaleOp;
#pragma unroll 1
  for (;;) {
    int k = 0;
#pragma unroll 1
    do {
      uint8_t* const cb = par ? buf1 : buf0;
      uint8_t* const nb_ = par ? buf0 : buf1;
      phase<true>(c, cb, 1, nb_, 1, dso_b, sso_b, f0, f1, sb, acc);
      phase<false>(c, nb_, 0, cb, 0, dso_a, sso_a, f1, f0, sa, acc);
      // blocks k + 3 (B) and k + 4 (A) for the next iteration
      dso_b = k + 3 == nb ? nxt.b : dso_b + 128u;
      sso_b = k + 3 == nb ? nxt.sb : sso_b + kScaleOp;
      dso_a = k + 4 == nb ? nxt.a : dso_a + 128u;
      sso_a = k + 4 == nb ? nxt.sa : sso_a + kScaleOp;
      par ^= 1;
      ++k;
    } while (k < nb);

    // lane holds Y[m0 + 128 wm + 16 q + rr][n0 + 128 wn + 16 i + 4 grp + 0..3]
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int m = cur.m0 + c.wm * 128 + q * 16 + rr;
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = cur.n0 + c.wn * 128 + i * 16 + 4 * grp;
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
    t += step;
    if (t >= ntiles) break;
    cur = nxt;
    nxt = tile_base(t + step < ntiles ? t + step : t, tiles_m, tiles_n, nb, krow);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // surplus staging loads
}

}  // namespace

namespace wush {

namespace {
// LDS kernel: 32-bit offsets (operands below 2 GiB) and at least two 128-wide
// K half-steps
bool use_lds_kernel(int M, int N, int K) {
  return static_cast<long>(M) * (K / 2) < (1L << 31) && static_cast<long>(N) * (K / 2) < (1L << 31) && K >= 256;
}

// Persistent form: whole 256-wide K blocks, at least four of them
bool use_persistent(int K) { return K % 256 == 0 && K / 256 >= 4; }

// Compute units of the current device (one persistent workgroup each),
// queried once per device.  (Concurrent first calls store the same value.)
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

// The LDS kernel on plane-ordered scales PA / PB: persistent when it applies
void launch_lds(int M, int N, int K, const uint8_t* A, const uint8_t* PA, const uint8_t* B, const uint8_t* PB,
                float* Y, long tiles, hipStream_t stream) {
  if (use_persistent(K)) {
    const long grid = std::min<long>(tiles, device_cus());
    hipLaunchKernelGGL(gemm_mxfp4_persist, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, A, PA, B, PB, Y,
                       M, N, K);
  } else {
    hipLaunchKernelGGL(gemm_mxfp4_lds, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, A, PA, B, PB, Y, M,
                       N, K);
  }
}
}  // namespace

// bytes of plane-ordered scales the LDS kernel needs (0 for the direct kernel)
size_t gemm_mxfp4_ws_bytes(int M, int N, int K) {
  if (M < 1 || N < 1 || K < 1 || !use_lds_kernel(M, N, K)) return 0;
  const size_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN, nb = (K + 255) / 256;
  return (tiles_m + tiles_n) * nb * kScaleOp;
}

// scales of one operand (rows x K/32 bytes, row-major) into plane order
wush_status mxfp4_scale_planes(int rows, int K, const uint8_t* S, uint8_t* P, hipStream_t stream) {
  const int tiles = (rows + kBM - 1) / kBM, nb = K / 256;
  hipLaunchKernelGGL(scales_to_planes, dim3(tiles, (nb + 1) / 2), dim3(256), 0, stream, S, rows,
                     static_cast<const uint8_t*>(nullptr), 0, tiles, K, nb, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_mxfp4_scale_planes launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

// the LDS kernel on scales already in plane order (K a multiple of 256)
wush_status gemm_mxfp4_planes(int M, int N, int K, const uint8_t* A, const uint8_t* PA, const uint8_t* B,
                              const uint8_t* PB, float* Y, hipStream_t stream) {
  if (!use_lds_kernel(M, N, K) || K % 256 != 0)
    return fail(WUSH_E_UNSUPPORTED, "wush_w4a4_gemm_mx_planes: needs K a multiple of 256 and operands below 2 GiB");
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  const long tiles = static_cast<long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffL) return fail(WUSH_E_SHAPE, "wush_w4a4_gemm_mx_planes: too many tiles");
  launch_lds(M, N, K, A, PA, B, PB, Y, tiles, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm_mx_planes launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

wush_status gemm_mxfp4(int M, int N, int K, const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                       float* Y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (use_lds_kernel(M, N, K)) {
    const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN, nb = (K + 255) / 256;
    const long tiles = static_cast<long>(tiles_m) * tiles_n;
    if (tiles > 0x7fffffffL || tiles_m > 65535 || tiles_n > 65535)
      return fail(WUSH_E_SHAPE, "wush_w4a4_gemm: too many tiles");
    // plane-ordered scales: the caller's workspace, else stream-ordered scratch
    const size_t pa_bytes = static_cast<size_t>(tiles_m) * nb * kScaleOp;
    const size_t p_bytes = gemm_mxfp4_ws_bytes(M, N, K);
    uint8_t* P = static_cast<uint8_t*>(ws);
    if (P) {
      if (ws_bytes < p_bytes) return fail(WUSH_E_ARG, "wush_w4a4_gemm: workspace of %zu bytes, need %zu", ws_bytes, p_bytes);
    } else {
      const hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&P), p_bytes, stream);
      if (e != hipSuccess)
        return fail(WUSH_E_HIP, "wush_w4a4_gemm scratch (%zu bytes): %s", p_bytes, hipGetErrorString(e));
    }
    hipLaunchKernelGGL(scales_to_planes, dim3(tiles_m + tiles_n, (nb + 1) / 2), dim3(256), 0, stream, SA, M, SB, N,
                       tiles_m, K, nb, P);
    launch_lds(M, N, K, A, P, B, P + pa_bytes, Y, tiles, stream);
    const hipError_t e = hipGetLastError();
    const hipError_t f = ws ? hipSuccess : hipFreeAsync(P, stream);
    if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm launch: %s", hipGetErrorString(e));
    if (f != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm scratch free: %s", hipGetErrorString(f));
    return WUSH_OK;
  }
  dim3 grid((N + kBlockN - 1) / kBlockN, (M + kBlockM - 1) / kBlockM);
  if (grid.y > 65535u) return fail(WUSH_E_SHAPE, "wush_w4a4_gemm: M=%d too large", M);
  hipLaunchKernelGGL(gemm_mxfp4_direct, grid, dim3(256), 0, stream, A, SA, B, SB, Y, M, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // namespace wush
