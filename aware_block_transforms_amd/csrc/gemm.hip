// wush_w4a4_gemm: argument checks and dispatch to the per-format kernels.
//
// "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization" (AI Radio):
// the W4A4 product of the transformed, quantized weights and activations; the
// WUSH news article (experiments paragraph) evaluates it for MXFP4, NVFP4 and
// INT4.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "common.h"

namespace wush {
size_t gemm_mxfp4_ws_bytes(int M, int N, int K);
wush_status gemm_mxfp4(int M, int N, int K, const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                       float* Y, void* ws, size_t ws_bytes, hipStream_t stream);
wush_status mxfp4_scale_planes(int rows, int K, const uint8_t* S, uint8_t* P, hipStream_t stream);
wush_status gemm_mxfp4_planes(int M, int N, int K, const uint8_t* A, const uint8_t* PA, const uint8_t* B,
                              const uint8_t* PB, float* Y, hipStream_t stream);
size_t gemm_nvfp4_ws_bytes(int M, int N, int K);
wush_status gemm_nvfp4(int M, int N, int K, const uint8_t* A, const uint8_t* SA, float ga, const uint8_t* B,
                       const uint8_t* SB, float gb, float* Y, void* ws, size_t ws_bytes, hipStream_t stream);
size_t gemm_int4_ws_bytes(int M, int N, int K);
wush_status gemm_int4(int M, int N, int K, const uint8_t* A, const uint16_t* SA, const uint8_t* B,
                      const uint16_t* SB, float* Y, void* ws, size_t ws_bytes, hipStream_t stream);
}  // namespace wush

extern "C" size_t wush_w4a4_gemm_ws_bytes(wush_format fmt, int M, int N, int K) {
  if (M < 1 || N < 1 || K < 128 || K % 128) return 0;
  if (fmt == WUSH_MXFP4) return wush::gemm_mxfp4_ws_bytes(M, N, K);
  if (fmt == WUSH_NVFP4) return wush::gemm_nvfp4_ws_bytes(M, N, K);
  if (fmt == WUSH_INT4) return wush::gemm_int4_ws_bytes(M, N, K);
  return 0;
}

extern "C" wush_status wush_w4a4_gemm(wush_format fmt, int M, int N, int K, const uint8_t* a_codes,
                                      const void* a_scales, float a_g, const uint8_t* b_codes, const void* b_scales,
                                      float b_g, float* Y, void* ws, size_t ws_bytes, void* stream) {
  if (wush_format_block(fmt) == 0) return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm: bad format %d", static_cast<int>(fmt));
  if (M < 1 || N < 1 || K < 128 || K % 128)
    return wush::fail(WUSH_E_SHAPE, "wush_w4a4_gemm: need M, N >= 1 and K a positive multiple of 128 (M=%d N=%d K=%d)",
                      M, N, K);
  if (!a_codes || !a_scales || !b_codes || !b_scales || !Y) return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm: null pointer");
  if (!wush::aligned16(a_codes) || !wush::aligned16(b_codes) || !wush::aligned16(Y) ||
      (reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(b_scales) & 3u))
    return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm: codes and Y must be 16-byte aligned, scales 4-byte aligned");
  if (ws && !wush::aligned16(ws)) return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm: workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (fmt) {
    case WUSH_MXFP4:
      return wush::gemm_mxfp4(M, N, K, a_codes, static_cast<const uint8_t*>(a_scales), b_codes,
                              static_cast<const uint8_t*>(b_scales), Y, ws, ws_bytes, s);
    case WUSH_NVFP4:
      if (!(a_g > 0.0f && a_g < 3.0e38f) || !(b_g > 0.0f && b_g < 3.0e38f))
        return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm: NVFP4 tensor scales must be positive and finite");
      return wush::gemm_nvfp4(M, N, K, a_codes, static_cast<const uint8_t*>(a_scales), a_g, b_codes,
                              static_cast<const uint8_t*>(b_scales), b_g, Y, ws, ws_bytes, s);
    case WUSH_INT4:
      return wush::gemm_int4(M, N, K, a_codes, static_cast<const uint16_t*>(a_scales), b_codes,
                             static_cast<const uint16_t*>(b_scales), Y, ws, ws_bytes, s);
  }
  return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm: bad format");
}

extern "C" wush_status wush_mxfp4_scale_planes(int rows, int K, const uint8_t* scales, uint8_t* planes,
                                               void* stream) {
  if (rows < 1 || K < 256 || K % 256 != 0)
    return wush::fail(WUSH_E_SHAPE, "wush_mxfp4_scale_planes: need rows >= 1 and K a multiple of 256");
  if (!scales || !planes) return wush::fail(WUSH_E_ARG, "wush_mxfp4_scale_planes: null pointer");
  if ((reinterpret_cast<uintptr_t>(scales) & 3u) || !wush::aligned16(planes))
    return wush::fail(WUSH_E_ARG, "wush_mxfp4_scale_planes: scales 4-byte and planes 16-byte aligned");
  return wush::mxfp4_scale_planes(rows, K, scales, planes, static_cast<hipStream_t>(stream));
}

extern "C" wush_status wush_w4a4_gemm_mx_planes(int M, int N, int K, const uint8_t* a_codes, const uint8_t* a_planes,
                                                const uint8_t* b_codes, const uint8_t* b_planes, float* Y,
                                                void* stream) {
  if (M < 1 || N < 1 || K < 256 || K % 256)
    return wush::fail(WUSH_E_SHAPE, "wush_w4a4_gemm_mx_planes: need M, N >= 1 and K a multiple of 256");
  if (!a_codes || !a_planes || !b_codes || !b_planes || !Y)
    return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm_mx_planes: null pointer");
  if (!wush::aligned16(a_codes) || !wush::aligned16(b_codes) || !wush::aligned16(Y) || !wush::aligned16(a_planes) ||
      !wush::aligned16(b_planes))
    return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm_mx_planes: codes, planes and Y must be 16-byte aligned");
  return wush::gemm_mxfp4_planes(M, N, K, a_codes, a_planes, b_codes, b_planes, Y, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// wush_w4a4_gemm_noalloc: the same matmul for callers that cannot allocate
// (code under graph capture, serving loops, harnesses that forbid hipMalloc).
// The scale re-layout goes to a fixed device array instead of a workspace.  In
// host code `scratch` names a host-side stand-in, not device memory, so the
// kernels only ever see the address hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.  Every call on a device shares
// that device's array; its pre-passes rewrite every byte the kernels read, so
// nothing needs clearing, and calls that overlap on one device race.

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];   // device address of `scratch` per device, once looked up

wush_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return wush::fail(WUSH_E_HIP, "wush_w4a4_gemm_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return wush::fail(WUSH_E_HIP, "wush_w4a4_gemm_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return wush::fail(WUSH_E_HIP, "wush_w4a4_gemm_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    scratch_dev[dev] = ptr;
  }
  *out = scratch_dev[dev];
  return WUSH_OK;
}

}  // namespace

extern "C" size_t wush_w4a4_gemm_noalloc_max_ws_bytes(void) { return kScratchBytes; }

extern "C" wush_status wush_w4a4_gemm_noalloc(wush_format fmt, int M, int N, int K, const uint8_t* a_codes,
                                              const void* a_scales, float a_g, const uint8_t* b_codes,
                                              const void* b_scales, float b_g, float* Y, void* stream) {
  if (wush_format_block(fmt) == 0)
    return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm_noalloc: bad format %d", static_cast<int>(fmt));
  if (M < 1 || N < 1 || K < 128 || K % 128)
    return wush::fail(WUSH_E_SHAPE,
                      "wush_w4a4_gemm_noalloc: need M, N >= 1 and K a positive multiple of 128 (M=%d N=%d K=%d)", M, N,
                      K);
  const size_t need = wush_w4a4_gemm_ws_bytes(fmt, M, N, K);
  if (need > kScratchBytes)
    return wush::fail(WUSH_E_SHAPE,
                      "wush_w4a4_gemm_noalloc: M=%d N=%d K=%d needs %zu bytes of scratch, above the fixed %zu",
                      M, N, K, need, kScratchBytes);
  if (!a_codes || !a_scales || !b_codes || !b_scales || !Y)
    return wush::fail(WUSH_E_ARG, "wush_w4a4_gemm_noalloc: null pointer");
  void* ws = nullptr;
  const wush_status st = scratch_for_current_device(&ws);
  if (st != WUSH_OK) return st;
  // never NULL here, so the general call cannot fall back to the memory pool
  return wush_w4a4_gemm(fmt, M, N, K, a_codes, a_scales, a_g, b_codes, b_scales, b_g, Y, ws, kScratchBytes, stream);
}
