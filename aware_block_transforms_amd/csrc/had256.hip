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
// vector maximum, an fp16 scale and codes in [-3, 3] stored as two bit planes.
//
// GEMV: instead of inverse-rotating every weight (8 butterflies per weight on
// the vector ALU), the rotation is moved to the activations, which every
// output row shares:  sum_k x_k * (s/16)(H q)_k = (s/16) * sum_m q_m (H x)_m
// because H is symmetric.  A pre-pass rotates each activation chunk once and
// splits it into two int8 terms; the weight stream then only unpacks codes to
// int8 (byte permutes) and the dot products run on the int8 matrix cores.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace {

constexpr int kVec = 256;
constexpr int kBytes = 96;

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

__global__ __launch_bounds__(kVec) void had256_pack_kernel(const float* __restrict__ W, int d_in,
                                                           uint8_t* __restrict__ planes,
                                                           uint16_t* __restrict__ scales) {
  __shared__ float v[kVec];
  __shared__ uint32_t wmax[kVec / 64];
  __shared__ uint8_t cc[kVec];
  const int t = threadIdx.x;
  const int nv = d_in / kVec;
  const size_t vec = blockIdx.x;                 // row * nv + chunk
  const size_t row = vec / nv, c = vec % nv;
  const float x = W[row * d_in + c * kVec + t];
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
  cc[t] = static_cast<uint8_t>(q & 7);
  __syncthreads();
  uint8_t* dst = planes + vec * kBytes;
  if (t < 64) {
    dst[t] = static_cast<uint8_t>((cc[4 * t] & 3) | ((cc[4 * t + 1] & 3) << 2) | ((cc[4 * t + 2] & 3) << 4) |
                                  ((cc[4 * t + 3] & 3) << 6));
  } else if (t < 96) {
    const int j = t - 64;
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) b |= ((cc[8 * j + i] >> 2) & 1u) << i;
    dst[t] = static_cast<uint8_t>(b);
  }
  if (t == 0) {
    uint16_t hb;
    __builtin_memcpy(&hb, &h, 2);
    scales[vec] = hb;
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
// with both sums exact in int32 (v_mfma_i32_16x16x64_i8), and
//   y[b][row] = sum_c (s / 16) * that, accumulated in fp32.
//
// K order.  The codes of a chunk are visited in an order that makes the
// 3-bit unpack cheap: lane group g (of the MFMA's four) owns codes 64 g ..
// 64 g + 63, i.e. bytes 16 g .. 16 g + 15 of the 2-bit plane and 64 + 8 g ..
// 64 + 8 g + 7 of the 1-bit plane (one 16-byte and one 8-byte load), and each
// int8 dword holds the codes 8 j + r of four consecutive octets j for one bit
// position r, so that both planes yield it with a shift and a mask.  Byte p of
// the lane's 16 MFMA-t operand bytes holds code
//   k = 8 (4 (2 g + qq) + jj) + 2 t + rr,  qq = p / 8, rr = (p / 4) % 2, jj = p % 4,
// and the pre-pass stores the activations in the same order.

constexpr int kGemvWaves = 4;      // K split inside a workgroup: wave w takes chunks w, w + 4, ...

// Pre-pass: one workgroup of 256 threads per (chunk, batch row).
// act: [nv][4 t][4 g][batch][16] int8, a_hi then (at + batch * d_in) a_lo.
__global__ __launch_bounds__(kVec) void had256_prep_kernel(const uint16_t* __restrict__ x, int batch, int d_in,
                                                           int8_t* __restrict__ act, float* __restrict__ sig) {
  __shared__ float v[kVec];
  __shared__ uint32_t wmax[kVec / 64];
  const int t = threadIdx.x, c = blockIdx.x, b = blockIdx.y;
  const int nv = d_in / kVec;
  const float xv = __uint_as_float(static_cast<uint32_t>(x[static_cast<size_t>(b) * d_in + c * kVec + t]) << 16);
  const float r = fwht256_lds(v, xv);
  uint32_t ab = __float_as_uint(r) & 0x7fffffffu;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ab = max(ab, static_cast<uint32_t>(__shfl_xor(static_cast<int>(ab), off)));
  if ((t & 63) == 0) wmax[t >> 6] = ab;
  __syncthreads();
  const float amax = __uint_as_float(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
  const float sigma = amax / 127.0f;
  int hi = 0, lo = 0;
  if (sigma > 0.0f) {
    const float u = r / sigma;
    hi = static_cast<int>(fminf(fmaxf(rintf(u), -127.0f), 127.0f));
    lo = static_cast<int>(fminf(fmaxf(rintf((u - static_cast<float>(hi)) * 128.0f), -127.0f), 127.0f));
  }
  // position of code k = t in the operand order described above
  const int j = t >> 3, rb = t & 7;
  const int q = j >> 2, jj = j & 3, g = q >> 1, qq = q & 1, tm = rb >> 1, rr = rb & 1;
  const int p = (2 * qq + rr) * 4 + jj;
  const size_t o = ((static_cast<size_t>(c * 4 + tm) * 4 + g) * batch + b) * 16 + p;
  act[o] = static_cast<int8_t>(hi);
  act[static_cast<size_t>(batch) * d_in + o] = static_cast<int8_t>(lo);
  if (t == 0) sig[static_cast<size_t>(b) * nv + c] = sigma;
}

typedef int v4i __attribute__((ext_vector_type(4)));

// The int8 codes of dword (qq, rr-bit position r) from the lane's plane data.
// lo_f / hi_f: 2-bit-plane bytes of the four octets (fields of codes 8j+0..3 /
// 8j+4..7); b2: 1-bit-plane bytes of the same octets.
__device__ __forceinline__ uint32_t codes4(uint32_t lo_f, uint32_t hi_f, uint32_t b2, int r) {
  const uint32_t src = (r < 4) ? lo_f : hi_f;
  const uint32_t l2 = (src >> (2 * (r & 3))) & 0x03030303u;
  const uint32_t h1 = (b2 >> r) & 0x01010101u;
  const uint32_t c = l2 | (h1 << 2);                       // 3-bit codes, one per byte
  return __builtin_amdgcn_perm(0xFFFEFDFCu, 0x03020100u, c);   // -> int8 in [-4, 3]
}

// Activation operands of chunk c for MFMA t = 0..3 (lane column n = r16 is
// batch row n; zero past nb), plus sigma.
__device__ __forceinline__ void load_act(const int8_t* __restrict__ act, const int8_t* __restrict__ act_lo,
                                         const float* __restrict__ sig, int c, int nv, int nb, int r16, int g,
                                         v4i (&ah)[4], v4i (&al)[4], float& sg) {
#pragma unroll
  for (int t = 0; t < 4; ++t) { ah[t] = v4i{0, 0, 0, 0}; al[t] = v4i{0, 0, 0, 0}; }
  sg = 0.0f;
  if (r16 < nb && c < nv) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const size_t o = ((static_cast<size_t>(c * 4 + t) * 4 + g) * nb + r16) * 16;
      ah[t] = *reinterpret_cast<const v4i*>(act + o);
      al[t] = *reinterpret_cast<const v4i*>(act_lo + o);
    }
    sg = sig[static_cast<size_t>(r16) * nv + c];
  }
}

// One workgroup = one 16-row tile.  Per pass of up to 16 chunks the tile's
// packed weights (16 rows x 96 B per chunk, contiguous in HBM) and scales are
// copied to LDS with full-line loads that are all in flight at once, then
// wave w takes chunks w, w + 4, ... of the pass out of LDS (rows padded to
// 1552 bytes: the 16 lanes of one row group hit distinct banks).  The
// activation operands (L2-resident) are loaded per chunk.
constexpr int kPassChunks = 16;
constexpr int kRowPitch = kPassChunks * kBytes + 16;   // 1552

template <int B>
__global__ __launch_bounds__(64 * kGemvWaves) void had256_gemv_i8_kernel(const int8_t* __restrict__ act,
                                                                         const float* __restrict__ sig,
                                                                         const uint8_t* __restrict__ planes,
                                                                         const uint16_t* __restrict__ scales,
                                                                         float* __restrict__ y, int nb, int d_out,
                                                                         int d_in) {
  // B is the compiled batch capacity; nb <= B rows of x / y are real.
  __shared__ __attribute__((aligned(16))) uint8_t wl[16 * kRowPitch];
  __shared__ uint16_t sl[16 * kPassChunks];
  __shared__ float red[kGemvWaves][16][B];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int nv = d_in / kVec;
  const int row0 = blockIdx.x * 16;
  const int8_t* act_lo = act + static_cast<size_t>(nb) * d_in;
  float yp[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int base = 0; base < nv; base += kPassChunks) {
    const int pc = min(kPassChunks, nv - base);           // chunks in this pass
    const int pieces = pc * (kBytes / 16);                 // 16-byte pieces per row
    // copy: piece i of row r (rows past d_out are zero)
    uint4 v[(16 * kPassChunks * kBytes / 16 + 64 * kGemvWaves - 1) / (64 * kGemvWaves)];
#pragma unroll
    for (int k = 0; k < static_cast<int>(sizeof(v) / sizeof(v[0])); ++k) {
      const int idx = tid + k * 64 * kGemvWaves;
      const int r = idx / pieces, pi = idx % pieces;
      v[k] = make_uint4(0u, 0u, 0u, 0u);
      if (r < 16 && row0 + r < d_out)
        v[k] = *reinterpret_cast<const uint4*>(planes + (static_cast<size_t>(row0 + r) * nv + base) * kBytes + pi * 16);
    }
    uint16_t sv = 0;
    const int sr = tid / kPassChunks, sc = tid % kPassChunks;
    if (tid < 16 * kPassChunks && sc < pc && row0 + sr < d_out) sv = scales[static_cast<size_t>(row0 + sr) * nv + base + sc];
#pragma unroll
    for (int k = 0; k < static_cast<int>(sizeof(v) / sizeof(v[0])); ++k) {
      const int idx = tid + k * 64 * kGemvWaves;
      const int r = idx / pieces, pi = idx % pieces;
      if (r < 16) *reinterpret_cast<uint4*>(wl + r * kRowPitch + pi * 16) = v[k];
    }
    if (tid < 16 * kPassChunks) sl[tid] = sv;
    __syncthreads();

    for (int cc = wave; cc < pc; cc += kGemvWaves) {
      const int c = base + cc;
      v4i ah[4], al[4];
      float sg;
      load_act(act, act_lo, sig, c, nv, nb, r16, g, ah, al, sg);
      const uint8_t* vp = wl + r16 * kRowPitch + cc * kBytes;
      const uint4 p1 = *reinterpret_cast<const uint4*>(vp + 16 * g);
      const uint2 p2 = *reinterpret_cast<const uint2*>(vp + 64 + 8 * g);
      // 2-bit-plane bytes of octets 4q .. 4q+3 for q = 2g + qq
      const uint32_t lo0 = __builtin_amdgcn_perm(p1.y, p1.x, 0x06040200u);
      const uint32_t hi0 = __builtin_amdgcn_perm(p1.y, p1.x, 0x07050301u);
      const uint32_t lo1 = __builtin_amdgcn_perm(p1.w, p1.z, 0x06040200u);
      const uint32_t hi1 = __builtin_amdgcn_perm(p1.w, p1.z, 0x07050301u);
      v4i dh = v4i{0, 0, 0, 0}, dl = v4i{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v4i w;
        w.x = static_cast<int>(codes4(lo0, hi0, p2.x, 2 * t));
        w.y = static_cast<int>(codes4(lo0, hi0, p2.x, 2 * t + 1));
        w.z = static_cast<int>(codes4(lo1, hi1, p2.y, 2 * t));
        w.w = static_cast<int>(codes4(lo1, hi1, p2.y, 2 * t + 1));
        dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, ah[t], dh, 0, 0, 0);
        dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, al[t], dl, 0, 0, 0);
      }
      // lane holds rows 4g + e of the tile for batch column r16
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        _Float16 hs;
        const uint16_t sb = sl[(4 * g + e) * kPassChunks + cc];
        __builtin_memcpy(&hs, &sb, 2);
        const float s = static_cast<float>(hs) * 0.0625f;
        yp[e] = fmaf(s * sg, fmaf(static_cast<float>(dl[e]), 0.0078125f, static_cast<float>(dh[e])), yp[e]);
      }
    }
    __syncthreads();
  }
  if (r16 < B) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][4 * g + e][r16] = yp[e];
  }
  __syncthreads();
  for (int i = tid; i < 16 * B; i += 64 * kGemvWaves) {
    const int rl = i / B, b = i % B, orow = row0 + rl;
    if (b < nb && orow < d_out) {
      float sum = red[0][rl][b];
#pragma unroll
      for (int w = 1; w < kGemvWaves; ++w) sum += red[w][rl][b];
      y[static_cast<size_t>(b) * d_out + orow] = sum;
    }
  }
}

template <int B>
void launch_gemv(int nb, int d_out, int d_in, const int8_t* act, const float* sig, const uint8_t* planes,
                 const uint16_t* scales, float* y, hipStream_t s) {
  hipLaunchKernelGGL(had256_gemv_i8_kernel<B>, dim3((d_out + 15) / 16), dim3(64 * kGemvWaves), 0, s, act, sig, planes,
                     scales, y, nb, d_out, d_in);
}

}  // namespace

extern "C" {

wush_status wush_had256_pack_weights(int d_out, int d_in, const float* W, uint8_t* planes, uint16_t* scales,
                                     void* stream) {
  if (d_out < 0 || d_in < kVec || d_in % kVec)
    return wush::fail(WUSH_E_SHAPE, "wush_had256_pack_weights: d_in must be a positive multiple of 256");
  if (d_out == 0) return WUSH_OK;
  if (!W || !planes || !scales) return wush::fail(WUSH_E_ARG, "wush_had256_pack_weights: null pointer");
  const size_t nvec = static_cast<size_t>(d_out) * (d_in / kVec);
  if (nvec > 0x7fffffffu) return wush::fail(WUSH_E_SHAPE, "wush_had256_pack_weights: too many vectors");
  hipLaunchKernelGGL(had256_pack_kernel, dim3(static_cast<unsigned>(nvec)), dim3(kVec), 0,
                     static_cast<hipStream_t>(stream), W, d_in, planes, scales);
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
  const size_t act = 2 * static_cast<size_t>(batch) * d_in;           // a_hi, a_lo
  return act + static_cast<size_t>(batch) * (d_in / kVec) * sizeof(float);   // sigma
}

wush_status wush_had256_gemv(int batch, int d_out, int d_in, const uint16_t* x, const uint8_t* planes,
                             const uint16_t* scales, float* y, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 1 || batch > 16 || d_out < 1 || d_in < kVec || d_in % kVec)
    return wush::fail(WUSH_E_SHAPE, "wush_had256_gemv: need 1 <= batch <= 16, d_out >= 1, d_in %% 256 == 0");
  if (!x || !planes || !scales || !y) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: null pointer");
  if (!wush::aligned16(planes)) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: planes must be 16-byte aligned");
  if (ws && !wush::aligned16(ws)) return wush::fail(WUSH_E_ARG, "wush_had256_gemv: workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
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
  float* sig = reinterpret_cast<float*>(wsp + act_bytes);
  hipLaunchKernelGGL(had256_prep_kernel, dim3(nv, batch), dim3(kVec), 0, s, x, batch, d_in, act, sig);
  if (batch == 1)
    launch_gemv<1>(batch, d_out, d_in, act, sig, planes, scales, y, s);
  else if (batch <= 4)
    launch_gemv<4>(batch, d_out, d_in, act, sig, planes, scales, y, s);
  else
    launch_gemv<16>(batch, d_out, d_in, act, sig, planes, scales, y, s);
  const hipError_t fe = ws ? hipSuccess : hipFreeAsync(wsp, s);
  if (fe != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_gemv scratch free: %s", hipGetErrorString(fe));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_had256_gemv launch: %s", hipGetErrorString(e));
  return WUSH_OK;
}

}  // extern "C"
