// NVFP4 x NVFP4 -> fp32 matmul for gfx950, LDS-staged.
//
// WUSH news article (chain.bitekongjian.com), experiments paragraph: the
// format sweep includes NVFP4 (16 E2M1 values sharing an E4M3 scale, and one
// fp32 scale per tensor).  CDNA4's block-scaled FP4 MFMA takes E8M0 scales
// per 32 values, so an NVFP4 block cannot ride on it.  Every product
// e2m1 * e4m3 has at most 6 significant bits and lies in [2^-10, 2688], so it
// is exact in fp16: the codes are dequantized to fp16 in registers and
// multiplied on the fp16 matrix cores (v_mfma_f32_16x16x32_f16, fp32
// accumulation); the two tensor scales multiply the result once.
//
// Decode: v_cvt_scalef32_pk_f16_fp4 turns two codes into fp16 (scale 1, so
// exact) and one v_pk_mul_f16 applies the block scale to the pair (exact, see
// above).  The conversion's own scale operand cannot carry an E4M3 scale: it
// applies only the exponent of its fp32 value.  One VALU operation per value
// keeps the vector ALU well inside the matrix-core time of a 128 x 128 wave
// tile.
//
// Tile: 256 x 256 per workgroup, four waves of 128 x 128 (256 AGPR
// accumulators), K in blocks of 256 staged through two LDS buffers with the
// XOR swizzle of the MXFP4 kernel.  Codes and scales go from HBM straight to
// LDS (buffer_load ... lds, one block ahead), so no VGPRs hold staging data;
// the scales are first re-laid by a pre-pass into the stage's plane order
// (4 KB per operand and block).  Each wave software-pipelines its decode: while
// the matrix cores run the eight MFMAs of one (K step, A fragment) group, the
// vector ALU decodes the next group's A fragment and one B fragment of the
// next K step, and the LDS reads of the next 128-wide sub-step are issued as
// the registers they replace die.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "common.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256;
constexpr int kFragOp = 16 * 2048;           // one operand of one block: 16 fragment pairs of 16 rows x 128 B
constexpr int kScaleOp = 16 * 256 * 2;       // one operand's scale planes per block (fp16)
constexpr int kStageBytes = 2 * kFragOp + 2 * kScaleOp;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw, unswizzled; dword 3 = 0x00020000 selects 32-bit data format for untyped access on CDNA
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
// s_waitcnt immediates (gfx9 layout), through the builtin so the compiler's
// own wait insertion knows what has completed
constexpr unsigned kWaitLgkm0 = 0xC07F;   // lgkmcnt(0)
constexpr unsigned kWaitVm0 = 0x0F70;     // vmcnt(0)

// All of this wave's LDS reads done, then the workgroup barrier; no memory
// fence (it would also wait for the DMA in flight).
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XCD-aware tile order (as in the MXFP4 kernel): workgroups are dealt to the
// 8 XCDs round-robin, each XCD gets a contiguous run of tiles walked in
// groups of kGroupM tile rows.
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

// Scales in plane order, as fp16 (every E4M3 value is an fp16 number, so
// the conversion is exact and the GEMM multiplies by them directly): for each
// 256-row tile t and 256-wide K block k, the 8 KB at (t nb + k) * 8192 hold 16
// planes p = (j * 4 + g) * 2 + e of 256 entries (sub-step j, lane K group g,
// half e of the lane's 32 values, i.e. NVFP4 block 2 (4 j + g) + e of the K
// block); entry [rr][pos] of a plane is the scale of tile row
// 128 (pos / 8) + 16 (pos % 8) + rr, with pos rotated by 8 for odd g
// (bank-conflict-free reads).  Zero past the operand and past K.  One
// workgroup of 256 threads (thread = tile row) per (block, tile).
__global__ __launch_bounds__(256) void nv_scales_to_planes(const uint8_t* __restrict__ SA, int ra,
                                                           const uint8_t* __restrict__ SB, int rb, int tiles_a,
                                                           int K, int nb, uint8_t* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) uint16_t planes[16 * 256];
  const int k = blockIdx.x, t = blockIdx.y, tr = threadIdx.x;
  const bool in_a = t < tiles_a;
  const int row = (in_a ? t : t - tiles_a) * kBM + tr;
  const int rows = in_a ? ra : rb;
  const int sdw = K / 64;   // scale dwords per row (K / 16 bytes)
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(in_a ? SA : SB) + static_cast<size_t>(row) * sdw;
  uint32_t v[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) v[d] = (row < rows && 4 * k + d < sdw) ? s32[4 * k + d] : 0u;
  const int rr = tr & 15, pos = 8 * (tr >> 7) + ((tr >> 4) & 7);
#pragma unroll
  for (int b16 = 0; b16 < 16; ++b16) {
    const int j = b16 >> 3, g = (b16 >> 1) & 3, e = b16 & 1;
    const int p = (j * 4 + g) * 2 + e;
    const int byte = static_cast<int>((v[b16 >> 2] >> (8 * (b16 & 3))) & 0xFFu);
    const _Float16 h = static_cast<_Float16>(__builtin_amdgcn_cvt_f32_fp8(byte, 0));
    planes[p * 256 + rr * 16 + (pos ^ (8 * (g & 1)))] = __builtin_bit_cast(uint16_t, h);
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(P + (static_cast<size_t>(t) * nb + k) * kScaleOp);
  dst[tr] = reinterpret_cast<const uint4*>(planes)[tr];
  dst[256 + tr] = reinterpret_cast<const uint4*>(planes)[256 + tr];
}

struct NvCtx {
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  uint32_t a_dma[2], b_dma[2];   // loader lane's byte offset within 8 rows x 128 B, for even / odd u
  uint32_t a_row0, b_row0;       // byte offset of the wave's first row (64 wave rows into the tile)
  uint32_t krow;                 // bytes per code row (K / 2)
  uint32_t sa_base, sb_base;     // byte offset of the tile's plane-ordered scales (block 0)
  uint32_t r_frag[2];            // LDS slot of this lane's read chunk within a fragment pair, per sub-step
  uint32_t r_scale_a, r_scale_b; // LDS offset of this lane's 8 fp16 scales within plane (j, g, e) = (0, g, 0)
  int wave, wm, wn;
};

typedef __attribute__((address_space(3))) void lds_void;

// DMA d (0..19) of this wave's share of block kb into stage buffer `buf`:
// d < 8: A codes rows 64 wave + 8 d .. + 7 (1 KB, a fragment pair's half);
// d < 16: the same for B; 16 .. 19: 1 KB halves of this wave's 2 KB of A's
// (16, 17) and B's (18, 19) scale planes.  LDS
// receives lane i's 16 bytes at offset 16 i, so each lane fetches the global
// chunk that the XOR swizzle puts in its slot.  Rows past the operand read as
// zeros (the bounds check covers the whole offset; their outputs are never
// stored); in a half block the upper 64 bytes of a row read the next row or
// zeros and feed only the skipped sub-step.
__device__ __forceinline__ void dma(const NvCtx& c, int d, int kb, uint8_t* buf) {
  const int lane = threadIdx.x & 63;
  if (d < 16) {
    const int op = d >> 3, u = d & 7;
    uint8_t* dst = buf + op * kFragOp + c.wave * (4 * 2048) + u * 1024;
    const uint32_t soff = (op ? c.b_row0 : c.a_row0) + static_cast<uint32_t>(8 * u) * c.krow + static_cast<uint32_t>(kb) * 128;
    const uint32_t voff = op ? c.b_dma[u & 1] : c.a_dma[u & 1];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? c.rb : c.ra, (lds_void*)(dst), 16, voff, soff, 0, 0);
  } else {
    const int op = (d - 16) >> 1, h = d & 1;
    uint8_t* dst = buf + 2 * kFragOp + op * kScaleOp + c.wave * 2048 + h * 1024;
    const uint32_t soff =
        (op ? c.sb_base : c.sa_base) + static_cast<uint32_t>(kb) * kScaleOp + c.wave * 2048 + h * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? c.rsb : c.rsa, (lds_void*)(dst), 16, lane * 16, soff, 0, 0);
  }
}

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) times the
// block scale (as an fp16 pair) -> 8 exact fp16 values.
__device__ __forceinline__ v8h decode8(uint32_t w, v2h s) {
  const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  return v8h{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ uint32_t word(const uint4& v, int t) {
  return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// fp16 scale number i of the eight in s, as a pair
__device__ __forceinline__ v2h half_pair(const uint4& s, int i) {
  const v2h w = __builtin_bit_cast(v2h, word(s, i >> 1));
  return (i & 1) ? v2h{w.y, w.y} : v2h{w.x, w.x};
}

// Registers carried from group to group: B decoded for the current K step
// (bc), A decoded for the current group (ad), the raw dwords the next two
// groups decode, and the scales of the current and the following sub-step
// (fp16, fragment i in half i; e = NVFP4 block within the lane's 32 values).
struct Regs {
  v8h bc[8];
  v8h ad;
  uint32_t rawa[2], rawb[2];   // for groups g + 1 (index 0) and g + 2 (index 1)
  uint4 sa[2], sb[2];           // fp16 scales of fragments 0..7, per block e
};

// Dword `t` of this lane's chunk of fragment f (operand op) of sub-step j.
__device__ __forceinline__ uint32_t read_word(const NvCtx& c, const uint8_t* buf, int op, int f, int j, int t) {
  const int row_pair = (op ? c.wn : c.wm) * 8 + f;
  return *reinterpret_cast<const uint32_t*>(buf + op * kFragOp + row_pair * 2048 + c.r_frag[j] + 4 * t);
}
__device__ __forceinline__ void read_scales(const NvCtx& c, const uint8_t* buf, int j, uint4 (&sa)[2], uint4 (&sb)[2]) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    sa[e] = *reinterpret_cast<const uint4*>(buf + 2 * kFragOp + (j * 8 + e) * 512 + c.r_scale_a);
    sb[e] = *reinterpret_cast<const uint4*>(buf + 2 * kFragOp + kScaleOp + (j * 8 + e) * 512 + c.r_scale_b);
  }
}

// What group g (t = g / 8, q = g % 8) of a sub-step decodes besides its MFMAs:
// the A operand of group g + 1 and B fragment q for K step t + 1 (for g >= 24
// and the last A these belong to the following sub-step).
struct Need { int af, at, bf, bt; bool a_next, b_next; };
__device__ __forceinline__ constexpr Need need_of(int g) {
  const int t = g >> 3, q = g & 7;
  Need n{0, 0, 0, 0, false, false};
  if (q < 7) { n.af = q + 1; n.at = t; }
  else if (t < 3) { n.af = 0; n.at = t + 1; }
  else { n.af = 0; n.at = 0; n.a_next = true; }
  n.bf = q;
  if (t < 3) n.bt = t + 1;
  else { n.bt = 0; n.b_next = true; }
  return n;
}

// One fp16 MFMA, D = C += B A, accumulator tied to its AGPR tuple.  Issued
// as inline asm: the compiler's own selection moves MFMA chains between
// register files when the loop carries 64 of them.  The asm is opaque to the
// compiler's hazard tracking, so the first MFMA of each group carries the
// wait states a VALU write of an operand needs before an MFMA reads it (every
// operand of a group is written in an earlier group).
template <bool kNop>
__device__ __forceinline__ void mfma(v4f& acc, const v8h& b, const v8h& a) {
  if (kNop)
    asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
  else
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

// The two codes of byte kSel of w as exact fp16 values.
template <int kSel>
__device__ __forceinline__ v2h cvt_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, kSel);
}


__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// One 128-wide K sub-step (sub-step j of buffer `buf`): 4 K steps t x 8 A
// fragments q; group (t, q) runs the eight fp16 MFMAs acc[i][q] += B_i(t)
// A_q(t).  Dword t of a lane's chunk holds K values 8 t .. 8 t + 7 of its 32,
// so MFMA step t of A and B pair the same K values; NVFP4 block e = t / 2 of
// the chunk.  Each group is laid out as eight slots of one MFMA and two or
// three vector operations (the wave issues in order, so the decode of the
// next operands must sit between the MFMAs to run while they do): the A
// operand of group g + 1, B fragment q of step t + 1, and the LDS reads of
// the raw dwords that group g + 2 decodes.  Reads for the following sub-step
// (nbuf, nj) start at group 22; the last read of this sub-step's own data
// is at group 28.
//   kBoundary: that sub-step starts a new block.  Group 22 waits for that
//          block's DMA and meets the other waves at a barrier before reading
//          it; group 29 meets them again, when no wave reads this block any
//          more, and groups 29-31 DMA block dma_k into `dma_buf` (the buffer
//          this block used; past the last block the caller passes the last
//          block again, which lands in a buffer no longer read: no branch
//          splits the MFMA stream).
// Sub-step state that lives across its groups.
struct SubState {
  uint4 nsa[2], nsb[2];   // the following sub-step's scales (read at group 22)
  v8h bn[8];              // B decoded for the next K step
};

// x times fp16 scale number kIdx of the eight in s (op_sel broadcast: free)
template <int kIdx>
__device__ __forceinline__ v2h mul_scale(v2h x, const uint4& s) {
  const v2h w = __builtin_bit_cast(v2h, word(s, kIdx >> 1));
  return (kIdx & 1) ? x * v2h{w.y, w.y} : x * v2h{w.x, w.x};
}

template <int g, bool kBoundary>
__device__ __forceinline__ void group(const NvCtx& c, Regs& r, SubState& ss, v4f (&acc)[8][8], const uint8_t* buf,
                                      int j, const uint8_t* nbuf, int nj, int dma_k, uint8_t* dma_buf) {
  constexpr int q = g & 7;
  constexpr Need nd = need_of(g);
  constexpr Need n2 = need_of((g + 2) & 31);
  constexpr bool g2_next = g + 2 >= 32;
  if (g == 22) {
    if (kBoundary) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      stage_barrier();
    }
    read_scales(c, nbuf, nj, ss.nsa, ss.nsb);
  }
  if (kBoundary && g == 29) stage_barrier();
  // the block's 20 DMAs after the second barrier: 7 per group in slots 0-6
  constexpr int d0 = 7 * (g - 29);
  const bool dma_here = kBoundary && g >= 29;
  // scales of this group's decodes: A operand of group g + 1, B fragment q
  // of the step after (both may belong to the following sub-step)
  const uint4& sa = nd.a_next ? ss.nsa[0] : r.sa[nd.at >> 1];
  const uint4& sb = nd.b_next ? ss.nsb[0] : r.sb[nd.bt >> 1];
  // Eight slots of one MFMA and two vector operations, software-pipelined so
  // that no slot waits on its own results (each conversion a slot ahead of
  // its multiply); the wave issues in order, so the decode must sit between
  // the MFMAs to run while they do.
  v2h ca0, ca1, ca2, ca3, cb0, cb1, cb2, cb3, pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3;
  uint32_t wa, wb;
  mfma<true>(acc[0][q], r.bc[0], r.ad);
  ca0 = cvt_pair<0>(r.rawa[0]);
  cb0 = cvt_pair<0>(r.rawb[0]);
  if (dma_here) dma(c, d0, dma_k, dma_buf);
  fence();
  mfma<false>(acc[1][q], r.bc[1], r.ad);
  ca1 = cvt_pair<1>(r.rawa[0]);
  pa0 = mul_scale<nd.af>(ca0, sa);
  if (dma_here) dma(c, d0 + 1, dma_k, dma_buf);
  fence();
  mfma<false>(acc[2][q], r.bc[2], r.ad);
  cb1 = cvt_pair<1>(r.rawb[0]);
  pb0 = mul_scale<q>(cb0, sb);
  {
    constexpr bool nx = g2_next || n2.a_next;
    wa = read_word(c, nx ? nbuf : buf, 0, n2.af, nx ? nj : j, n2.at);
  }
  if (dma_here) dma(c, d0 + 2, dma_k, dma_buf);
  fence();
  mfma<false>(acc[3][q], r.bc[3], r.ad);
  ca2 = cvt_pair<2>(r.rawa[0]);
  pa1 = mul_scale<nd.af>(ca1, sa);
  if (dma_here && d0 + 3 < 20) dma(c, d0 + 3, dma_k, dma_buf);
  fence();
  mfma<false>(acc[4][q], r.bc[4], r.ad);
  cb2 = cvt_pair<2>(r.rawb[0]);
  pb1 = mul_scale<q>(cb1, sb);
  if (dma_here && d0 + 4 < 20) dma(c, d0 + 4, dma_k, dma_buf);
  fence();
  mfma<false>(acc[5][q], r.bc[5], r.ad);
  ca3 = cvt_pair<3>(r.rawa[0]);
  pa2 = mul_scale<nd.af>(ca2, sa);
  {
    constexpr bool nx = g2_next || n2.b_next;
    wb = read_word(c, nx ? nbuf : buf, 1, n2.bf, nx ? nj : j, n2.bt);
  }
  if (dma_here && d0 + 5 < 20) dma(c, d0 + 5, dma_k, dma_buf);
  fence();
  mfma<false>(acc[6][q], r.bc[6], r.ad);
  cb3 = cvt_pair<3>(r.rawb[0]);
  pb2 = mul_scale<q>(cb2, sb);
  if (dma_here && d0 + 6 < 20) dma(c, d0 + 6, dma_k, dma_buf);
  fence();
  mfma<false>(acc[7][q], r.bc[7], r.ad);
  pa3 = mul_scale<nd.af>(ca3, sa);
  pb3 = mul_scale<q>(cb3, sb);
  fence();
  r.ad = v8h{pa0.x, pa0.y, pa1.x, pa1.y, pa2.x, pa2.y, pa3.x, pa3.y};
  ss.bn[q] = v8h{pb0.x, pb0.y, pb1.x, pb1.y, pb2.x, pb2.y, pb3.x, pb3.y};
  r.rawa[0] = r.rawa[1];
  r.rawb[0] = r.rawb[1];
  r.rawa[1] = wa;
  r.rawb[1] = wb;
  if (q == 7) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r.bc[i] = ss.bn[i];
  }
}

template <bool kBoundary, int... G>
__device__ __forceinline__ void groups(const NvCtx& c, Regs& r, SubState& ss, v4f (&acc)[8][8], const uint8_t* buf,
                                       int j, const uint8_t* nbuf, int nj, int dma_k, uint8_t* dma_buf,
                                       std::integer_sequence<int, G...>) {
  (group<G, kBoundary>(c, r, ss, acc, buf, j, nbuf, nj, dma_k, dma_buf), ...);
}

template <bool kBoundary>
__device__ __forceinline__ void sub_step(const NvCtx& c, Regs& r, v4f (&acc)[8][8], const uint8_t* buf, int j,
                                         const uint8_t* nbuf, int nj, int dma_k, uint8_t* dma_buf) {
  SubState ss;
  groups<kBoundary>(c, r, ss, acc, buf, j, nbuf, nj, dma_k, dma_buf, std::make_integer_sequence<int, 32>{});
  r.sa[0] = ss.nsa[0];
  r.sa[1] = ss.nsa[1];
  r.sb[0] = ss.nsb[0];
  r.sb[1] = ss.nsb[1];
}

__global__ __launch_bounds__(256, 1) void gemm_nvfp4_lds(const uint8_t* __restrict__ A, const uint8_t* __restrict__ PA,
                                                        const uint8_t* __restrict__ B, const uint8_t* __restrict__ PB,
                                                        float gab, float* __restrict__ Y, int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];
  NvCtx c;
  const int tid = threadIdx.x, lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.wm = c.wave >> 1;
  c.wn = c.wave & 1;
  const int nb = (K + 255) / 256;
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int rr = lane & 15, grp = lane >> 4;
  // 32-bit offsets (the host checks the operands are below 2^31 bytes)
  c.krow = static_cast<uint32_t>(K) / 2;
  const int lr = lane >> 3, lc = lane & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // slot lc of row lr + 8 h of a fragment pair holds chunk lc ^ ((row / 2) % 8)
    const uint32_t v = static_cast<uint32_t>(lr) * c.krow + ((lc ^ (((lr + 8 * h) >> 1) & 7)) * 16);
    c.a_dma[h] = v;
    c.b_dma[h] = v;
  }
  c.a_row0 = static_cast<uint32_t>(m0 + 64 * c.wave) * c.krow;
  c.b_row0 = static_cast<uint32_t>(n0 + 64 * c.wave) * c.krow;
  c.sa_base = static_cast<uint32_t>(tm * nb) * kScaleOp;
  c.sb_base = static_cast<uint32_t>(tn * nb) * kScaleOp;
#pragma unroll
  for (int j = 0; j < 2; ++j) c.r_frag[j] = rr * 128 + ((((4 * j + grp) ^ ((rr >> 1) & 7))) * 16);
  // odd K groups keep their planes rotated by 8 bytes (disjoint banks)
  c.r_scale_a = grp * 1024 + 2 * (rr * 16 + ((c.wm * 8) ^ (8 * (grp & 1))));
  c.r_scale_b = grp * 1024 + 2 * (rr * 16 + ((c.wn * 8) ^ (8 * (grp & 1))));
  c.ra = make_rsrc(A, static_cast<uint32_t>(M) * c.krow);
  c.rb = make_rsrc(B, static_cast<uint32_t>(N) * c.krow);
  c.rsa = make_rsrc(PA, static_cast<uint32_t>(tiles_m * nb) * kScaleOp);
  c.rsb = make_rsrc(PB, static_cast<uint32_t>(tiles_n * nb) * kScaleOp);

  // Each accumulator starts as its own AGPR tuple: left as one shared zero,
  // the loop's accumulator copies cannot be coalesced and every MFMA pays
  // for register shuffles.
  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      acc[i][q] = v4f{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[i][q]));
    }

  uint8_t* const buf0 = smem;
  uint8_t* const buf1 = smem + kStageBytes;
  // prologue: block 0 into buffer 0 and published; block 1 on its way into
  // buffer 1; sub-step 0's first operands decoded, the raw dwords of its
  // groups 0 and 1 read
#pragma unroll
  for (int d = 0; d < 20; ++d) dma(c, d, 0, buf0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  stage_barrier();
#pragma unroll
  for (int d = 0; d < 20; ++d) dma(c, d, min(1, nb - 1), buf1);
  Regs r;
  read_scales(c, buf0, 0, r.sa, r.sb);
#pragma unroll
  for (int i = 0; i < 8; ++i) r.bc[i] = decode8(read_word(c, buf0, 1, i, 0, 0), half_pair(r.sb[0], i));
  r.ad = decode8(read_word(c, buf0, 0, 0, 0, 0), half_pair(r.sa[0], 0));
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const Need n = need_of(g);
    r.rawa[g] = read_word(c, buf0, 0, n.af, 0, n.at);
    r.rawb[g] = read_word(c, buf0, 1, n.bf, 0, n.bt);
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_sched_barrier(0);

  // Every block runs both sub-steps, so one copy of the code serves all: in a
  // half block (K % 256 = 128) the second sub-step's scales are the zeros the
  // pre-pass writes past K, so it adds exact zeros; after the last block the
  // prefetch reads stale LDS into registers that are never used.  (A
  // do-while: with a loop that may run zero times the accumulators are not
  // carried through the loop in their own registers.)
  int k = 0;
#pragma unroll 1
  do {
    uint8_t* cur = (k & 1) ? buf1 : buf0;
    uint8_t* oth = (k & 1) ? buf0 : buf1;
    sub_step<false>(c, r, acc, cur, 0, cur, 1, 0, nullptr);
    sub_step<true>(c, r, acc, cur, 1, oth, 0, min(k + 2, nb - 1), cur);
    ++k;
  } while (k < nb);
  // no DMA may still be writing this workgroup's LDS when it exits; the last
  // MFMAs' results are ready before anything reads the accumulators (the asm
  // MFMAs are invisible to the compiler's hazard tracking)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) asm volatile("" : "+a"(acc[i][q]));

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
        *reinterpret_cast<float4*>(dst) =
            make_float4(acc[i][q][0] * gab, acc[i][q][1] * gab, acc[i][q][2] * gab, acc[i][q][3] * gab);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) dst[e] = acc[i][q][e] * gab;
      }
    }
  }
}

bool use_nv_lds(int M, int N, int K) {
  return static_cast<long>(M) * (K / 2) < (1L << 31) && static_cast<long>(N) * (K / 2) < (1L << 31);
}

}  // namespace

namespace wush {

wush_status gemm_nvfp4_direct(int M, int N, int K, const uint8_t* A, const uint8_t* SA, float ga, const uint8_t* B,
                              const uint8_t* SB, float gb, float* Y, hipStream_t stream);

size_t gemm_nvfp4_ws_bytes(int M, int N, int K) {
  if (M < 1 || N < 1 || K < 1 || !use_nv_lds(M, N, K)) return 0;
  const size_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN, nb = (K + 255) / 256;
  return (tiles_m + tiles_n) * nb * kScaleOp;
}

wush_status gemm_nvfp4(int M, int N, int K, const uint8_t* A, const uint8_t* SA, float ga, const uint8_t* B,
                       const uint8_t* SB, float gb, float* Y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!use_nv_lds(M, N, K)) return gemm_nvfp4_direct(M, N, K, A, SA, ga, B, SB, gb, Y, stream);
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN, nb = (K + 255) / 256;
  const long tiles = static_cast<long>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffffL || tiles_m + tiles_n > 65535 || nb > 65535)
    return fail(WUSH_E_SHAPE, "wush_w4a4_gemm (nvfp4): too many tiles");
  const size_t pa_bytes = static_cast<size_t>(tiles_m) * nb * kScaleOp;
  const size_t p_bytes = gemm_nvfp4_ws_bytes(M, N, K);
  uint8_t* P = static_cast<uint8_t*>(ws);
  if (P) {
    if (ws_bytes < p_bytes) return fail(WUSH_E_ARG, "wush_w4a4_gemm: workspace of %zu bytes, need %zu", ws_bytes, p_bytes);
  } else {
    const hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&P), p_bytes, stream);
    if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm scratch (%zu bytes): %s", p_bytes, hipGetErrorString(e));
  }
  hipLaunchKernelGGL(nv_scales_to_planes, dim3(nb, tiles_m + tiles_n), dim3(256), 0, stream, SA, M, SB, N, tiles_m, K,
                     nb, P);
  hipLaunchKernelGGL(gemm_nvfp4_lds, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, A, P, B, P + pa_bytes,
                     ga * gb, Y, M, N, K);
  const hipError_t e = hipGetLastError();
  const hipError_t f = ws ? hipSuccess : hipFreeAsync(P, stream);
  if (e != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm (nvfp4) launch: %s", hipGetErrorString(e));
  if (f != hipSuccess) return fail(WUSH_E_HIP, "wush_w4a4_gemm scratch free: %s", hipGetErrorString(f));
  return WUSH_OK;
}

}  // namespace wush
