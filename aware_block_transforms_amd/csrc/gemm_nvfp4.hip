// NVFP4 x NVFP4 -> fp32 matmul for gfx950, LDS-staged.
//
// WUSH news article (chain.bitekongjian.com), experiments paragraph: the
// format sweep includes NVFP4 (16 E2M1 values sharing an E4M3 scale, and one
// fp32 scale per tensor).  CDNA4's block-scaled FP4 MFMA takes E8M0 scales
// per 32 values, so an NVFP4 block cannot ride on it.  Every product
// e2m1 * e4m3 has at most 6 significant bits and lies in [2^-10, 2688], so it
// is exact in fp16: the codes are dequantized to fp16 in registers and
// multiplied on the fp16 matrix cores (v_mfma_f32_32x32x16_f16, fp32
// accumulation); the two tensor scales multiply the result once.
//
// Decode: v_cvt_scalef32_pk_f16_fp4 turns two codes into fp16 (scale 1, so
// exact) and one v_pk_mul_f16 applies the block scale to the pair (exact, see
// above), broadcast from an fp16 copy of the scales through op_sel.  The
// conversion's own scale operand cannot carry an E4M3 scale: it applies only
// the exponent of its fp32 value.
//
// Tile: 256 x 256 per workgroup, four waves of 128 x 128 (4 x 4 MFMAs of
// 32 x 32, 256 AGPR accumulators), K in blocks of 256 staged through two LDS
// buffers of 80 KB.  Codes and the pre-pass's re-laid fp16 scales go from HBM
// straight to LDS (buffer_load ... lds, one block ahead), so no VGPRs hold
// staging data.  The wave issues in order and an MFMA plus four vector
// operations fill one 32 x 32 MFMA's time, so each K step of 16 MFMAs carries
// the decode of the next step's eight operands between them (two conversions
// and two multiplies per MFMA), and each lane reads its raw codes as whole
// 16-byte chunks, two per operand and 128-wide sub-step.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "common.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kCodeOp = 256 * 128;          // one operand of one block: 256 rows x 128 B of codes
constexpr int kScaleOp = 16 * 256 * 2;       // one operand's scales per block (fp16)
constexpr int kStageBytes = 2 * kCodeOp + 2 * kScaleOp;
constexpr int kGroupM = 4;
constexpr int kXcds = 8;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

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
// treat it as an LDS store: its own wait insertion would then make every
// later LDS read wait for all DMA in flight.  The kernel orders the two
// itself (s_waitcnt vmcnt(0) and a barrier before LDS written by DMA is
// read).  The instruction writes no register except M0, which nothing
// else in these kernels reads (a CPU test checks the compiled code).
__device__ __forceinline__ void dma16(const v4i& desc, const void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
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

// Scales re-laid as fp16 (every E4M3 value is an fp16 number, so the
// conversion is exact and the GEMM multiplies by them directly).  For each
// 256-row tile and 256-wide K block, 8 KB: entry
//   ((((j * 2 + h) * 2 + w) * 2 + x) * 32 + r) * 8 + (e & 1) * 4 + f
// holds the scale of tile row 128 w + 32 f + r for NVFP4 block 8 j + 4 h + e
// of the K block (sub-step j, lane half h, e = 2 x + (e & 1)): the eight
// scales a lane needs for one pair of K steps are 16 contiguous bytes, and
// consecutive lanes read consecutive 16-byte pieces.  Zero past the operand
// and past K.  One workgroup of 256 threads (thread = tile row) per (block,
// tile); tiles 0 .. tiles_a - 1 come from SA (ra rows), the rest from SB.
__global__ __launch_bounds__(256) void nv_scales_to_planes(const uint8_t* __restrict__ SA, int ra,
                                                           const uint8_t* __restrict__ SB, int rb, int tiles_a,
                                                           int K, int nb, uint8_t* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) uint16_t planes[kScaleOp / 2];
  const int k = blockIdx.x, t = blockIdx.y, tr = threadIdx.x;
  const bool in_a = t < tiles_a;
  const int row = (in_a ? t : t - tiles_a) * kBM + tr;
  const int rows = in_a ? ra : rb;
  const int sdw = K / 64;   // scale dwords per row (K / 16 bytes)
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(in_a ? SA : SB) + static_cast<size_t>(row) * sdw;
  uint32_t v[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) v[d] = (row < rows && 4 * k + d < sdw) ? s32[4 * k + d] : 0u;
  const int w = tr >> 7, f = (tr >> 5) & 3, r = tr & 31;
#pragma unroll
  for (int b16 = 0; b16 < 16; ++b16) {
    const int j = b16 >> 3, h = (b16 >> 2) & 1, e = b16 & 3;
    const int idx = ((((j * 2 + h) * 2 + w) * 2 + (e >> 1)) * 32 + r) * 8 + (e & 1) * 4 + f;
    const int byte = static_cast<int>((v[b16 >> 2] >> (8 * (b16 & 3))) & 0xFFu);
    planes[idx] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(__builtin_amdgcn_cvt_f32_fp8(byte, 0)));
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(P + (static_cast<size_t>(t) * nb + k) * kScaleOp);
  dst[tr] = reinterpret_cast<const uint4*>(planes)[tr];
  dst[256 + tr] = reinterpret_cast<const uint4*>(planes)[256 + tr];
}

struct NvCtx {
  v4i ra, rb, rsa, rsb;           // buffer descriptors of A, B and the re-laid scales
  uint32_t a_dma[2], b_dma[2];   // loader lane's byte offset within 8 rows x 128 B, for even / odd u
  uint32_t a_row0, b_row0;       // byte offset of the wave's first loaded row (64 wave rows into the tile)
  uint32_t krow;                 // bytes per code row (K / 2)
  uint32_t sa_base, sb_base;     // byte offset of the tile's re-laid scales (block 0)
  uint32_t r_code[2][2];         // LDS offset of this lane's chunk [sub-step j][half] within its fragment
  uint32_t r_scale_a, r_scale_b; // LDS offset of this lane's scales for (j, x) = (0, 0)
  int wave, wm, wn;
};

// DMA d (0..19) of this wave's share of block kb into stage buffer `buf`:
// d < 8: A codes rows 64 wave + 8 d .. + 7 (1 KB); d < 16: the same for B;
// 16 .. 19: 1 KB halves of this wave's 2 KB of A's (16, 17) and B's (18, 19)
// re-laid scales.  LDS receives lane i's 16 bytes at offset 16 i, so each
// lane fetches the global chunk that the XOR swizzle puts in its slot.  Rows
// past the operand read as zeros (the bounds check covers the whole offset;
// their outputs are never stored); in a half block the upper 64 bytes of a
// row read the next row or zeros, multiplied by the zero scales past K.
__device__ __forceinline__ void dma(const NvCtx& c, int d, int kb, uint8_t* buf) {
  const int lane = threadIdx.x & 63;
  if (d < 16) {
    const int op = d >> 3, u = d & 7;
    uint8_t* dst = buf + op * kCodeOp + c.wave * (64 * 128) + u * 1024;
    const uint32_t soff = (op ? c.b_row0 : c.a_row0) + static_cast<uint32_t>(8 * u) * c.krow + static_cast<uint32_t>(kb) * 128;
    const uint32_t voff = op ? c.b_dma[u & 1] : c.a_dma[u & 1];
    dma16(op ? c.rb : c.ra, dst, voff, soff);
  } else {
    const int op = (d - 16) >> 1, h = d & 1;
    uint8_t* dst = buf + 2 * kCodeOp + op * kScaleOp + c.wave * 2048 + h * 1024;
    const uint32_t soff =
        (op ? c.sb_base : c.sa_base) + static_cast<uint32_t>(kb) * kScaleOp + c.wave * 2048 + h * 1024;
    dma16(op ? c.rsb : c.rsa, dst, lane * 16, soff);
  }
}

__device__ __forceinline__ uint32_t word(const uint4& v, int t) {
  return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// The two codes of byte kSel of w as exact fp16 values.
template <int kSel>
__device__ __forceinline__ v2h cvt_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, kSel);
}

// x times fp16 scale number kIdx of the eight in s (op_sel broadcast: free)
template <int kIdx>
__device__ __forceinline__ v2h mul_scale(v2h x, const uint4& s) {
  const v2h w = __builtin_bit_cast(v2h, word(s, kIdx >> 1));
  return (kIdx & 1) ? x * v2h{w.y, w.y} : x * v2h{w.x, w.x};
}

// One fp16 MFMA 32x32x16, D = C += B A, accumulator tied to its AGPR tuple.
// Issued as inline asm: the compiler's own selection moves MFMA chains between
// register files when a loop carries 16 of them.  The asm is opaque to the
// compiler's hazard tracking; every operand is written at least four
// instructions before an MFMA reads it (the decode schedule below), and the
// accumulators are read only after the wait that follows the loop.
__device__ __forceinline__ void mfma32(v16f& acc, const v8h& b, const v8h& a) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// v with values 2 p, 2 p + 1 replaced by x
template <int p>
__device__ __forceinline__ v8h put(v8h v, v2h x) {
  const v8h w = __builtin_shufflevector(x, x, 0, 1, 0, 1, 0, 1, 0, 1);
  if constexpr (p == 0) return __builtin_shufflevector(v, w, 8, 9, 2, 3, 4, 5, 6, 7);
  else if constexpr (p == 1) return __builtin_shufflevector(v, w, 0, 1, 8, 9, 4, 5, 6, 7);
  else if constexpr (p == 2) return __builtin_shufflevector(v, w, 0, 1, 2, 3, 8, 9, 6, 7);
  else return __builtin_shufflevector(v, w, 0, 1, 2, 3, 4, 5, 8, 9);
}

// Wave state carried from slot to slot.  Operand o < 4 is B fragment o (32
// weight rows), o >= 4 is A fragment o - 4 (32 activation rows); a lane holds
// row r = lane % 32 of each and, per 128-wide sub-step, the 64 K values of
// half h = lane / 32: two 16-byte chunks, "lo" (K steps 0-3) and "hi" (4-7),
// dword s % 4 being K step s.
struct State {
  uint4 lo[8], hi[8];        // raw code chunks
  uint4 sa[2], sb[2];        // fp16 scales of this sub-step: [x] holds (e & 1) * 4 + f for e = 2 x + (e & 1)
  uint4 nsa[2], nsb[2];      // the same for the following sub-step
  v8h cur[8];                // decoded operands of the current K step
  v8h nxt[8];                // the next K step's, being decoded
  v2h cv[2];                 // converted pairs waiting for their multiply
};

// raw dword and fp16 scale of operand o for K step t (t = 8: the following
// sub-step's step 0, whose lo chunks and scales have been read by then)
template <int o, int t>
__device__ __forceinline__ uint32_t raw_of(const State& st) {
  if constexpr ((t & 7) < 4) return word(st.lo[o], t & 3);
  else return word(st.hi[o], t & 3);
}
template <int o, int t, int p>
__device__ __forceinline__ v2h scaled(const State& st, v2h x) {
  constexpr int e = (t & 7) >> 1, idx = (e & 1) * 4 + (o & 3);
  if constexpr (o < 4) {
    if constexpr (t == 8) return mul_scale<idx>(x, st.nsb[e >> 1]);
    else return mul_scale<idx>(x, st.sb[e >> 1]);
  } else {
    if constexpr (t == 8) return mul_scale<idx>(x, st.nsa[e >> 1]);
    else return mul_scale<idx>(x, st.sa[e >> 1]);
  }
}

__device__ __forceinline__ const uint8_t* code_at(const NvCtx& c, const uint8_t* buf, int o, int j, int half) {
  const int op = o < 4 ? 1 : 0, f = o & 3;
  const int w = op ? c.wn : c.wm;
  return buf + op * kCodeOp + (128 * w + 32 * f) * 128 + c.r_code[j][half];
}
__device__ __forceinline__ void read_scales(const NvCtx& c, const uint8_t* buf, int j, uint4 (&sa)[2], uint4 (&sb)[2]) {
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    sa[x] = *reinterpret_cast<const uint4*>(buf + 2 * kCodeOp + c.r_scale_a + (j * 8 + x) * 512);
    sb[x] = *reinterpret_cast<const uint4*>(buf + 2 * kCodeOp + kScaleOp + c.r_scale_b + (j * 8 + x) * 512);
  }
}

// Slot z of K step s of a sub-step (sub-step j of buffer `buf`): one MFMA
// acc[z % 4][z / 4] += B_{z%4}(s) A_{z/4}(s), then two multiplies (the pairs
// converted in the previous slot) and two conversions of the next step's
// operands: operand z / 2, pairs 2 (z % 2) and 2 (z % 2) + 1.  The wave issues
// in order, so the decode sits between the MFMAs to run while they do; each
// conversion is multiplied a slot later, so no slot waits on its own results.
// The last pairs of A fragment 3 are multiplied in slot 0 of the step that
// uses them (first read in slot 12).  LDS reads: the hi chunks in step 1, the
// following sub-step's lo chunks and scales (nbuf, nj) in step 5.
//   kBoundary: the following sub-step starts a new block.  Slot (5, 0) waits
//          for that block's DMA and meets the other waves at a barrier: by then
//          no wave reads this block any more (its last reads are the step-1 hi
//          chunks) and the next block has landed; then 20 DMAs bring block
//          dma_k into `dma_buf` (the buffer this block used; past the last
//          block the caller passes the last block again, which lands in a
//          buffer no longer read: no branch splits the MFMA stream).
template <int s, int z, bool kBoundary>
__device__ __forceinline__ void slot(const NvCtx& c, State& st, v16f (&acc)[4][4], const uint8_t* buf, int j,
                                     const uint8_t* nbuf, int nj, int dma_k, uint8_t* dma_buf) {
  if (kBoundary && s == 5 && z == 0) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stage_barrier();
  }
  mfma32(acc[z & 3][z >> 2], st.cur[z & 3], st.cur[4 + (z >> 2)]);
  // multiplies of the previous slot's conversions
  if (z == 0) {
    st.cur[7] = put<2>(st.cur[7], scaled<7, s, 2>(st, st.cv[0]));
    st.cur[7] = put<3>(st.cur[7], scaled<7, s, 3>(st, st.cv[1]));
  } else {
    constexpr int P = 2 * z - 2, o = P >> 2, p = P & 3;
    st.nxt[o] = put<p>(st.nxt[o], scaled<o, s + 1, p>(st, st.cv[0]));
    st.nxt[o] = put<p + 1>(st.nxt[o], scaled<o, s + 1, p + 1>(st, st.cv[1]));
  }
  // conversions for the next K step
  {
    constexpr int o = z >> 1, p = 2 * (z & 1);
    const uint32_t w = raw_of<o, s + 1>(st);
    st.cv[0] = cvt_pair<p>(w);
    st.cv[1] = cvt_pair<p + 1>(w);
  }
  if (s == 1 && z < 8) st.hi[z] = *reinterpret_cast<const uint4*>(code_at(c, buf, z, j, 1));
  if (s == 5 && z < 8) st.lo[z] = *reinterpret_cast<const uint4*>(code_at(c, nbuf, z, nj, 0));
  if (s == 5 && z == 8) read_scales(c, nbuf, nj, st.nsa, st.nsb);
  if (kBoundary && s == 5 && z >= 1) dma(c, z - 1, dma_k, dma_buf);
  if (kBoundary && s == 6 && z < 5) dma(c, 15 + z, dma_k, dma_buf);
  fence();
  if (z == 15) {
#pragma unroll
    for (int o = 0; o < 8; ++o) st.cur[o] = st.nxt[o];   // A fragment 3's last pairs follow in slot 0
  }
}

template <bool kBoundary, int... I>
__device__ __forceinline__ void slots(const NvCtx& c, State& st, v16f (&acc)[4][4], const uint8_t* buf, int j,
                                      const uint8_t* nbuf, int nj, int dma_k, uint8_t* dma_buf,
                                      std::integer_sequence<int, I...>) {
  (slot<I / 16, I % 16, kBoundary>(c, st, acc, buf, j, nbuf, nj, dma_k, dma_buf), ...);
}

template <bool kBoundary>
__device__ __forceinline__ void sub_step(const NvCtx& c, State& st, v16f (&acc)[4][4], const uint8_t* buf, int j,
                                         const uint8_t* nbuf, int nj, int dma_k, uint8_t* dma_buf) {
  slots<kBoundary>(c, st, acc, buf, j, nbuf, nj, dma_k, dma_buf, std::make_integer_sequence<int, 128>{});
  st.sa[0] = st.nsa[0];
  st.sa[1] = st.nsa[1];
  st.sb[0] = st.nsb[0];
  st.sb[1] = st.nsb[1];
}

template <int o, int p>
__device__ __forceinline__ v2h first_pair(const State& st) {
  return scaled<o, 0, p>(st, cvt_pair<p>(word(st.lo[o], 0)));
}
template <int... O>
__device__ __forceinline__ void decode_first(State& st, std::integer_sequence<int, O...>) {
  ((st.cur[O >> 2] = put<(O & 3)>(st.cur[O >> 2], first_pair<(O >> 2), (O & 3)>(st))), ...);
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
  const int r = lane & 31, h = lane >> 5;
  // 32-bit offsets (the host checks the operands are below 2^31 bytes)
  c.krow = static_cast<uint32_t>(K) / 2;
  const int lr = lane >> 3, lc = lane & 7;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    // slot lc of tile row R holds chunk lc ^ ((R / 2) % 8); loader rows are 64 wave + 8 u + lr
    const uint32_t v = static_cast<uint32_t>(lr) * c.krow + ((lc ^ (((lr + 8 * hh) >> 1) & 7)) * 16);
    c.a_dma[hh] = v;
    c.b_dma[hh] = v;
  }
  c.a_row0 = static_cast<uint32_t>(m0 + 64 * c.wave) * c.krow;
  c.b_row0 = static_cast<uint32_t>(n0 + 64 * c.wave) * c.krow;
  c.sa_base = static_cast<uint32_t>(tm * nb) * kScaleOp;
  c.sb_base = static_cast<uint32_t>(tn * nb) * kScaleOp;
  // a lane reads chunk 4 j + 2 h + half of row 128 w + 32 f + r, whose slot is
  // that index ^ ((r / 2) % 8) (128 w + 32 f is a multiple of 16)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int half = 0; half < 2; ++half)
      c.r_code[j][half] = r * 128 + (((4 * j + 2 * h + half) ^ ((r >> 1) & 7)) * 16);
  // scale entry (j, h, w, x, r): (((j 2 + h) 2 + w) 2 + x) 32 + r, 16 bytes each
  c.r_scale_a = (((h * 2 + c.wm) * 2) * 32 + r) * 16;
  c.r_scale_b = (((h * 2 + c.wn) * 2) * 32 + r) * 16;
  c.ra = make_desc(A, static_cast<uint32_t>(M) * c.krow);
  c.rb = make_desc(B, static_cast<uint32_t>(N) * c.krow);
  c.rsa = make_desc(PA, static_cast<uint32_t>(tiles_m * nb) * kScaleOp);
  c.rsb = make_desc(PB, static_cast<uint32_t>(tiles_n * nb) * kScaleOp);

  // Each accumulator starts as its own AGPR tuple: left as one shared zero,
  // the loop's accumulator copies cannot be coalesced.
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[i][q] = v16f{};
      asm volatile("" : "+a"(acc[i][q]));
    }

  uint8_t* const buf0 = smem;
  uint8_t* const buf1 = smem + kStageBytes;
  // prologue: block 0 into buffer 0 and published; block 1 on its way into
  // buffer 1; sub-step 0's lo chunks and scales read and its step-0 operands
  // decoded (the last two pairs of A fragment 3 left converted, as slot
  // (0, 0) expects)
#pragma unroll
  for (int d = 0; d < 20; ++d) dma(c, d, 0, buf0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  stage_barrier();
#pragma unroll
  for (int d = 0; d < 20; ++d) dma(c, d, min(1, nb - 1), buf1);
  State st;
#pragma unroll
  for (int o = 0; o < 8; ++o) st.lo[o] = *reinterpret_cast<const uint4*>(code_at(c, buf0, o, 0, 0));
  read_scales(c, buf0, 0, st.sa, st.sb);
  decode_first(st, std::make_integer_sequence<int, 30>{});
  st.cv[0] = cvt_pair<2>(word(st.lo[7], 0));
  st.cv[1] = cvt_pair<3>(word(st.lo[7], 0));
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("s_nop 4" ::: "memory");   // wait states between the decode above and the first MFMA
  fence();

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
    sub_step<false>(c, st, acc, cur, 0, cur, 1, 0, nullptr);
    sub_step<true>(c, st, acc, cur, 1, oth, 0, min(k + 2, nb - 1), cur);
    ++k;
  } while (k < nb);
  // no DMA may still be writing this workgroup's LDS when it exits; the last
  // MFMAs' results are ready before anything reads the accumulators (the asm
  // MFMAs are invisible to the compiler's hazard tracking)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : "+a"(acc[i][q]));

  // lane holds Y[m0 + 128 wm + 32 q + r][n0 + 128 wn + 32 i + 8 p + 4 h + 0..3]
  // in acc[i][q][4 p .. 4 p + 3]
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = m0 + c.wm * 128 + q * 32 + r;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int n = n0 + c.wn * 128 + i * 32 + 8 * p + 4 * h;
        float* dst = Y + static_cast<size_t>(m) * N + n;
        const float v0 = acc[i][q][4 * p] * gab, v1 = acc[i][q][4 * p + 1] * gab;
        const float v2 = acc[i][q][4 * p + 2] * gab, v3 = acc[i][q][4 * p + 3] * gab;
        if (n + 3 < N && (N & 3) == 0) {
          *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
        } else {
          if (n < N) dst[0] = v0;
          if (n + 1 < N) dst[1] = v1;
          if (n + 2 < N) dst[2] = v2;
          if (n + 3 < N) dst[3] = v3;
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
