/*
 * wush.h - C ABI of libwush: data-aware block transforms (WUSH) followed by
 * low-bit block quantization and a W4A4 matmul, native to AMD Instinct MI355X
 * (gfx950 / CDNA4).
 *
 * Sources (web pages, cited by title and section):
 *  [WUSH-news]  "WUSH" news article (chain.bitekongjian.com): paragraphs on
 *               the construction, on optimality, on experiments (MXFP4,
 *               NVFP4, INT4) and on the deployment workflow.
 *  [WUSH-radio] "WUSH: Near-Optimal Adaptive Transforms for LLM
 *               Quantization" (AI Radio episode): "Problem Setup and Goal"
 *               (layer loss), "The gist" (fused GPU implementation).
 *  [ITQ3_S]     ITQ3_S article (ai.866data.com): "Core technique: FWHT
 *               pre-rotation" section.
 *
 * Conventions shared by every call
 *  - Layouts are row-major.  Weights use the nn.Linear layout Wt[d_out][d_in]
 *    (the transpose of the pages' W, which is d_in x d_out); activations are
 *    token-major Xt[n][d_in] (the transpose of the pages' X).  Block b covers
 *    input channels [b*bs, (b+1)*bs); transforms and quantization groups both
 *    run along d_in (the reduction dimension K of the matmul).
 *  - Packed 4-bit codes: byte j of a row holds element 2j in its low nibble
 *    and element 2j+1 in its high nibble.
 *  - The caller owns every buffer.  "Device" pointers are plain HIP device
 *    allocations (for example torch tensors' data_ptr()); "host" pointers are
 *    ordinary CPU memory.  Device pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Device calls are asynchronous on that stream unless stated otherwise;
 *    faults during execution surface at the caller's next synchronisation.
 *  - Every call validates its arguments before launching anything and returns
 *    a wush_status; nothing aborts or throws across the ABI.  The thread-local
 *    string returned by wush_last_error() describes the most recent failure.
 *  - Calls keep no global mutable state besides that string and are safe to
 *    call from several threads on different streams.
 */
#ifndef WUSH_H
#define WUSH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WUSH_OK = 0,
  WUSH_E_ARG = 1,          /* null pointer, bad enum, misaligned pointer   */
  WUSH_E_SHAPE = 2,        /* sizes that do not divide / exceed limits      */
  WUSH_E_NUMERIC = 3,      /* Cholesky failed after damping; non-finite g   */
  WUSH_E_HIP = 4,          /* a HIP runtime call or launch failed           */
  WUSH_E_UNSUPPORTED = 5   /* valid request this build does not implement   */
} wush_status;

/* Block formats named for the experiments of [WUSH-news]. */
typedef enum {
  WUSH_MXFP4 = 0,  /* 32 E2M1 values + one E8M0 scale byte                    */
  WUSH_NVFP4 = 1,  /* 16 E2M1 values + one E4M3 scale byte, fp32 tensor scale */
  WUSH_INT4 = 2    /* 32 symmetric int4 values in [-7,7] + one fp16 scale     */
} wush_format;

/* Transform families compared in [WUSH-news] (experiments paragraph). */
typedef enum {
  WUSH_IDENTITY = 0,
  WUSH_HADAMARD = 1,  /* orthonormal Sylvester Hadamard H/sqrt(bs)        */
  WUSH_WUS = 2,       /* S^{1/2} U^T W'^{-1} (no Hadamard factor)          */
  WUSH_WUSH = 3       /* H/sqrt(bs) S^{1/2} U^T W'^{-1}                    */
} wush_kind;

typedef enum { WUSH_F32 = 0, WUSH_BF16 = 1 } wush_dtype;

/* Block size of a format: 32 (MXFP4, INT4) or 16 (NVFP4); 0 for a bad value. */
int wush_format_block(wush_format fmt);

/* ------------------------------------------------------------------------
 * Offline, host (CPU, fp64 inside, synchronous; no device memory touched).
 * ---------------------------------------------------------------------- */

/* Activation second moments per block, [WUSH-news] deployment paragraph
 * (moments come from calibration data):  Sx[b] = X_b X_b^T / n.
 *   X   host, [n][d_in] fp32 (token-major calibration activations).
 *   Sx  host out, [d_in/bs][bs][bs] fp32 (accumulated in fp64, rounded once).
 * Errors: WUSH_E_ARG (null), WUSH_E_SHAPE (n < 1, bs not 16/32, d_in % bs). */
wush_status wush_block_moments(int bs, int n, int d_in, const float* X, float* Sx);

/* The same moments on the GPU (device pointers, stream-ordered): the step
 * before the builder, [WUSH-news] deployment paragraph (moments from
 * calibration data; per-block work in parallel).  Products are formed exactly
 * in fp64 and summed in fp64 per chunk of up to 256 tokens, the chunks in
 * order, then divided by n and rounded once to fp32; Sx is exactly symmetric.
 * Agrees with wush_block_moments up to fp64 summation order.
 *   X   device, [n][d_in] fp32 or bf16 (xdt), 16-byte aligned.
 *   Sx  device out, [d_in/bs][bs][bs] fp32.
 *   ws  device scratch of wush_block_moments_dev_ws_bytes(bs, n, d_in) bytes
 *       (fp64 chunk partials, 16-byte aligned), or NULL (taken from the
 *       default memory pool for the call).
 * Errors: WUSH_E_ARG, WUSH_E_SHAPE (n < 1, bs not 16/32, d_in % bs), WUSH_E_HIP. */
size_t wush_block_moments_dev_ws_bytes(int bs, int n, int d_in);
wush_status wush_block_moments_dev(int bs, wush_dtype xdt, int n, int d_in, const void* X,
                                   float* Sx, void* ws, size_t ws_bytes, void* stream);

/* Per-block transform pair, [WUSH-news] construction paragraph (Cholesky
 * factor of weight statistics, U and S of an SVD, Hadamard) and deployment
 * paragraph (per block, in parallel).  For every block b:
 *   A_b = W_b W_b^T (fp64, summed over the d_out rows),  A_b = W' W'^T,
 *   C_b = W'^T Sx_b W' = U diag(lambda) U^T (lambda descending, each column
 *   of U signed so its largest-magnitude entry is positive), S = sqrt(lambda),
 *   T_W = Q S^{1/2} U^T W'^{-1},  T_X = Q S^{-1/2} U^T W'^T = T_W^{-T},
 *   with Q = H/sqrt(bs) for WUSH and Q = I for WUS.  IDENTITY and HADAMARD
 *   ignore W and Sx (which may then be NULL).  If A_b is not positive
 *   definite the Cholesky is retried on A_b + eps*(tr A_b/bs)*I for
 *   eps = 1e-10, 1e-8, 1e-6, 1e-4, 1e-2; sigma_i is floored at 1e-12*sigma_1.
 *   W   host, [d_out][d_in] fp32.        Sx  host, [d_in/bs][bs][bs] fp32.
 *   Tx, Tw  host out, [d_in/bs][bs][bs] fp32 row-major (y = T x per block).
 * Errors: WUSH_E_ARG, WUSH_E_SHAPE (bs not 16/32, d_in % bs), WUSH_E_NUMERIC
 * (a block still not positive definite after the damping ladder). */
wush_status wush_build_transforms(wush_kind kind, int bs, int d_in, int d_out,
                                  const float* W, const float* Sx, float* Tx, float* Tw);

/* MXFP4 scales in the matmul's plane order.  wush_w4a4_gemm first rewrites
 * both operands' row-major E8M0 scales into the order its LDS stage keeps
 * them (a pre-pass per call).  These calls let a caller do that once for the
 * weights (wush_mxfp4_scale_planes, offline), have the activation step write
 * that order directly (wush_transform_quant_mx_planes), and run the matmul on
 * both (wush_w4a4_gemm_mx_planes): same kernels, bit-identical Y.
 * Layout (K a multiple of 256): 2048 bytes per (256-row tile t, 256-wide K
 * block kb) at (t * K/256 + kb) * 2048; within it, the scale of row
 * r = row % 256 and group b = (k / 32) % 8 sits at
 *   256 b + 16 (r % 16) + ((8 (r / 128) + (r / 16) % 8) XOR 8 (b % 2)).
 * Bytes of rows past `rows` are zero after wush_mxfp4_scale_planes and left
 * untouched by wush_transform_quant_mx_planes (the matmul never stores those
 * rows).  wush_mxfp4_planes_bytes(rows, K) is the buffer size (0 for bad
 * shapes).
 *   wush_transform_quant_mx_planes: wush_transform_quant for MXFP4 with
 *     scales written to `planes` in this layout; d_in % 256 == 0; Tx not NULL.
 *   wush_w4a4_gemm_mx_planes: Y = A W^T as wush_w4a4_gemm (MXFP4) from the
 *     plane-ordered scales; K % 256 == 0 and operands below 2 GiB, else
 *     WUSH_E_SHAPE / WUSH_E_UNSUPPORTED.  Codes, planes and Y 16-byte aligned. */
size_t wush_mxfp4_planes_bytes(int rows, int K);
wush_status wush_mxfp4_scale_planes(int rows, int K, const uint8_t* scales, uint8_t* planes,
                                    void* stream);
wush_status wush_transform_quant_mx_planes(wush_dtype xdt, int n, int d_in, const void* X,
                                           const float* Tx, uint8_t* codes, uint8_t* planes,
                                           void* stream);
wush_status wush_w4a4_gemm_mx_planes(int M, int N, int K, const uint8_t* a_codes,
                                     const uint8_t* a_planes, const uint8_t* b_codes,
                                     const uint8_t* b_planes, float* Y, void* stream);

/* wush_build_transforms on the GPU ([WUSH-news] deployment paragraph: the
 * per-block computations are independent and parallel).  Same construction,
 * operation order and fp64 arithmetic as the host call, so the two produce
 * the same matrices; W and Sx (for instance from wush_block_moments_dev) stay
 * on the device.  Offline: one thread per block for the factorisations.
 *   W, Sx   device, as in wush_build_transforms (unused for IDENTITY/HADAMARD).
 *   Tx, Tw  device out, [d_in/bs][bs][bs] fp32.
 *   ws      device workspace of wush_build_transforms_dev_ws_bytes(bs, d_in)
 *           bytes (fp64 weight moments and per-block status), 16-byte aligned.
 * Synchronises `stream` (the damping results come back to the host).
 * Errors: those of wush_build_transforms, plus WUSH_E_ARG for a missing or
 * short workspace and WUSH_E_HIP. */
size_t wush_build_transforms_dev_ws_bytes(int bs, int d_in);
wush_status wush_build_transforms_dev(wush_kind kind, int bs, int d_in, int d_out,
                                      const float* W, const float* Sx, float* Tx, float* Tw,
                                      void* ws, size_t ws_bytes, void* stream);

/* Shared-transform variant ([WUSH-news], paragraph on deployment limits:
 * similar blocks share one transform).  The caller assigns each block b a
 * group group[b] in [0, ngroups); every group must own a block.  A group's
 * matrices are those of wush_build_transforms for the group's summed moments
 *   A_G = sum_{b in G} W_b W_b^T,  B_G = sum_{b in G} Sx_b   (fp64, block order),
 * (a reading: the pages give no construction for the shared matrix).
 *   group   host, [d_in/bs] int32.
 *   Tx, Tw  host out, [ngroups][bs][bs] fp32.
 * Errors: those of wush_build_transforms; WUSH_E_ARG for a group id out of
 * range or an empty group. */
wush_status wush_build_shared(wush_kind kind, int bs, int d_in, int d_out, const float* W,
                              const float* Sx, int ngroups, const int* group, float* Tx,
                              float* Tw);

/* Hadamard-diagonal variant ([WUSH-news], deployment and limitation
 * paragraphs: the data-aware component approximated by a diagonal matrix).
 * Reading: the construction above with the moments replaced by their
 * diagonals.  Per block b and channel i: a_i = sum_o W[o][i]^2 (fp64) and
 * s_i = Sx_b[i][i]; values below 1e-12 of their block's largest are raised to
 * that floor (s_i = 1 when the block's s are all zero);
 *   dx_i = f32(sqrt(sqrt(a_i / s_i)) / sqrt(bs)),
 *   dw_i = f32(sqrt(sqrt(s_i / a_i)) / sqrt(bs)),
 * so T_X = H diag(dx) and T_W = H diag(dw) = T_X^{-T} (H the +-1 Sylvester
 * matrix): among Hadamard-times-diagonal pairs the one that minimises the
 * proxy loss, (sum_i sqrt(a_i s_i))^2.
 *   W   host, [d_out][d_in] fp32.      Sx  host, [d_in/bs][bs][bs] fp32.
 *   dx, dw  host out, [d_in] fp32 each.
 * Errors: WUSH_E_ARG, WUSH_E_SHAPE (bs not 16/32, d_in % bs, d_out < 1),
 * WUSH_E_NUMERIC (a block whose weights are all zero). */
wush_status wush_build_hd(int bs, int d_in, int d_out, const float* W, const float* Sx,
                          float* dx, float* dw);

/* ------------------------------------------------------------------------
 * Device calls (HIP, gfx950).
 * ---------------------------------------------------------------------- */

/* Transform then quantize activations: the online step of [WUSH-news]
 * (deployment paragraph: only activations are transformed at inference),
 * fused as in [WUSH-radio] "The gist".  Per token and block:
 *   y_i = fma chain over k ascending from +0 of T[i][k]*x[k] (fp32; T == NULL
 *   means the identity transform, a bit-exact copy), then the block quantizer:
 *   MXFP4: a = max|y|, e = clamp(floor(log2 a) - 2, -127, 127) (a == 0 -> -127),
 *          scale byte e+127, codes E2M1(y * 2^-e);
 *   NVFP4: s8 = E4M3(min(f32(a / f32(6g)), 448)), s = f32(dec(s8) * g),
 *          codes E2M1(f32(y * f32(1/s))) (all 0 if s == 0);
 *   INT4:  s16 = fp16(f32(a/7)), codes clamp(rint(f32(y * f32(1/s16))), -7, 7) & 15
 *          (all 0 if s16 == 0).
 *   E2M1 rounds to nearest, ties to the even code, saturates at 6 and copies the
 *   sign bit.  A block with a NaN/Inf value gets the format's NaN scale (0xFF,
 *   0x7F, 0x7E00) and all-zero codes.
 *   X       device, [n][d_in] fp32 or bf16 (xdt).
 *   Tx      device, [d_in/bs][bs][bs] fp32, or NULL for identity (16-byte aligned).
 *   g       NVFP4 per-tensor fp32 scale (> 0, finite); ignored otherwise.
 *   codes   device out, [n][d_in/2] bytes.
 *   scales  device out, [n][d_in/bs]: uint8 (MXFP4, NVFP4) or uint16 fp16 bits (INT4).
 * Errors: WUSH_E_ARG, WUSH_E_SHAPE (n < 0, d_in % bs), WUSH_E_HIP. */
wush_status wush_transform_quant(wush_format fmt, wush_dtype xdt, int n, int d_in,
                                 const void* X, const float* Tx, float g,
                                 uint8_t* codes, void* scales, void* stream);

/* The transform of wush_transform_quant without the quantizer: Y = T x per
 * token and block ([WUSH-news] deployment paragraph), with the same pinned
 * fp32 FMA chain, so Y holds exactly the values the quantizers see.
 *   bs      16 or 32.          X   device, [n][d_in] fp32 or bf16 (xdt).
 *   Tx      device, [d_in/bs][bs][bs] fp32 (not NULL, 16-byte aligned).
 *   Y       device out, [n][d_in] fp32.  X and Y 16-byte aligned.
 * Errors: WUSH_E_ARG, WUSH_E_SHAPE, WUSH_E_HIP. */
wush_status wush_transform_apply(wush_dtype xdt, int bs, int n, int d_in, const void* X,
                                 const float* Tx, float* Y, void* stream);

/* NVFP4 per-tensor scale of transformed data: g = f32(max|T x| / 2688)
 * (2688 = 6 * 448, the largest E2M1 value times the largest E4M3 value).
 * Used on calibration activations; the weight path computes it itself.
 * Synchronises `stream`; *g_out is a host pointer.  bs is 16.
 * Errors: WUSH_E_ARG, WUSH_E_SHAPE, WUSH_E_HIP, WUSH_E_NUMERIC (non-finite
 * or zero maximum). */
wush_status wush_nvfp4_global_scale(wush_dtype xdt, int n, int d_in, const void* X,
                                    const float* Tx, float* g_out, void* stream);

/* Transform and quantize weights offline ([WUSH-news] deployment paragraph:
 * weights are transformed once, after training): the same arithmetic as
 * wush_transform_quant with T_W applied to every weight row.  For NVFP4 the
 * per-tensor scale is computed first (wush_nvfp4_global_scale on the rows)
 * and written to *g_out (host pointer; the call then synchronises `stream`);
 * g_out may be NULL for the other formats.
 *   W       device, [d_out][d_in] fp32.     Tw  device, [d_in/bs][bs][bs] fp32 or NULL.
 *   codes   device out, [d_out][d_in/2].    scales  device out, [d_out][d_in/bs]. */
wush_status wush_pack_weights(wush_format fmt, int d_out, int d_in, const float* W,
                              const float* Tw, uint8_t* codes, void* scales,
                              float* g_out, void* stream);

/* The shared-transform variant of the three calls above (matrices from
 * wush_build_shared): block b of every row is transformed with group[b]'s
 * matrix, with the same pinned arithmetic, quantizers, outputs and errors.
 *   Tx / Tw  device, [ngroups][bs][bs] fp32, 16-byte aligned (not NULL).
 *   group    device, [d_in/bs] int32; ids outside [0, ngroups) are clamped to
 *            that range (no out-of-bounds read), so pass valid ids. */
wush_status wush_transform_quant_shared(wush_format fmt, wush_dtype xdt, int n, int d_in,
                                        const void* X, const float* Tx, int ngroups,
                                        const int* group, float g, uint8_t* codes,
                                        void* scales, void* stream);
wush_status wush_nvfp4_global_scale_shared(wush_dtype xdt, int n, int d_in, const void* X,
                                           const float* Tx, int ngroups, const int* group,
                                           float* g_out, void* stream);
wush_status wush_pack_weights_shared(wush_format fmt, int d_out, int d_in, const float* W,
                                     const float* Tw, int ngroups, const int* group,
                                     uint8_t* codes, void* scales, float* g_out, void* stream);

/* The Hadamard-diagonal variant of the three calls above (scales from
 * wush_build_hd, device pointers, [d_in] fp32).  The transform per token (or
 * weight row) and block is pinned as: v_k = f32(x_k * d_k), then butterfly
 * stages h = 1, 2, ..., bs/2, each pair (j, j + h) with j in the lower half of
 * a 2h-aligned group becoming (v_j + v_{j+h}, v_j - v_{j+h}) in fp32 (no
 * fused multiply-add).  Quantizers, outputs, NVFP4 tensor scale, ownership and
 * errors are those of wush_transform_quant, wush_nvfp4_global_scale and
 * wush_pack_weights. */
wush_status wush_transform_quant_hd(wush_format fmt, wush_dtype xdt, int n, int d_in,
                                    const void* X, const float* dx, float g,
                                    uint8_t* codes, void* scales, void* stream);
wush_status wush_nvfp4_global_scale_hd(wush_dtype xdt, int n, int d_in, const void* X,
                                       const float* dx, float* g_out, void* stream);
wush_status wush_pack_weights_hd(wush_format fmt, int d_out, int d_in, const float* W,
                                 const float* dw, uint8_t* codes, void* scales,
                                 float* g_out, void* stream);

/* W4A4 matmul, the "FP4 MatMul" of [WUSH-radio]:
 *   Y[m][j] = sum_k dec(A)[m][k] * dec(B)[j][k],  fp32 output, fp32 accumulation.
 * dec() multiplies each code by its block scale (and by a_g / b_g for NVFP4).
 *   A: a_codes [M][K/2], a_scales [M][K/bs]  (activations, from wush_transform_quant)
 *   B: b_codes [N][K/2], b_scales [N][K/bs]  (weights, from wush_pack_weights)
 *   Y: device out, [M][N] fp32.
 *   ws: device scratch of at least wush_w4a4_gemm_ws_bytes(fmt, M, N, K)
 *       bytes (16-byte aligned), used only during the call (stream order);
 *       calls that share a ws must be ordered on one stream.  ws = NULL makes
 *       the call take the scratch itself from the device's default memory pool
 *       (hipMallocAsync / hipFreeAsync on `stream`), which costs several
 *       microseconds per call.
 * MXFP4 runs on the gfx950 block-scaled FP4 matrix cores (K >= 256 first
 * re-lays the scales, in ws, in the order the kernel stages them).  NVFP4
 * dequantizes exactly to fp16 (every E2M1 x E4M3 product is an fp16 number)
 * on the fp16 matrix cores, its block scales likewise re-laid in ws first.
 * INT4 runs one exact int8 matrix product per 32-group with an fp32 rescale,
 * its scales re-laid as fp32 in ws first.  The workspace size is 0 where a
 * path needs none (operands of 2^31 bytes or more take slower direct-load
 * kernels without scratch).  Asynchronous on
 * `stream`; A and B are only read.
 * Errors: WUSH_E_ARG (null or misaligned pointers, ws_bytes too small),
 * WUSH_E_SHAPE (M, N < 1; K < 1 or K % 128), WUSH_E_HIP (launch failure, or no
 * scratch from the pool). */
size_t wush_w4a4_gemm_ws_bytes(wush_format fmt, int M, int N, int K);
wush_status wush_w4a4_gemm(wush_format fmt, int M, int N, int K,
                           const uint8_t* a_codes, const void* a_scales, float a_g,
                           const uint8_t* b_codes, const void* b_scales, float b_g,
                           float* Y, void* ws, size_t ws_bytes, void* stream);

/* wush_w4a4_gemm without allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result and errors as wush_w4a4_gemm
 * except ws: the scale re-layout goes to a fixed 16 MiB device array that the
 * library holds on every device it runs on until the process ends
 * (wush_w4a4_gemm_noalloc_max_ws_bytes()).  Shapes whose
 * wush_w4a4_gemm_ws_bytes exceed it return WUSH_E_SHAPE before anything is
 * launched (MXFP4 fits both Qwen3-14B MLP projections at 16384 tokens; NVFP4
 * and INT4 fit the 4096 x 4096 x 8192-token square).  Calls no hipMalloc or
 * hipFree.  All calls on one device share its array: calls that overlap on
 * that device (two streams, two threads) race and must be ordered by the
 * caller.  The stream must belong to the current device. */
size_t wush_w4a4_gemm_noalloc_max_ws_bytes(void);
wush_status wush_w4a4_gemm_noalloc(wush_format fmt, int M, int N, int K,
                                   const uint8_t* a_codes, const void* a_scales, float a_g,
                                   const uint8_t* b_codes, const void* b_scales, float b_g,
                                   float* Y, void* stream);

/* Layer loss of [WUSH-radio] "Problem Setup and Goal":
 *   *loss = sum over M x N of (Yhat - Yref)^2 / (M * N), accumulated in fp64
 *   with a fixed two-stage reduction order (deterministic).
 *   Yhat, Yref device, [M][N] fp32; loss device out (one double);
 *   ws device workspace of wush_loss_ws_bytes(M, N) bytes. */
wush_status wush_layer_loss(int M, int N, const float* Yhat, const float* Yref,
                            double* loss, void* ws, void* stream);
size_t wush_loss_ws_bytes(int M, int N);

/* ------------------------------------------------------------------------
 * Hadamard-256 3-bit weight-only path ([ITQ3_S], core-technique section:
 * 256-point Walsh-Hadamard pre-rotation before a uniform 3-bit quantizer,
 * inverse rotation when weights are loaded for the matmul).
 * ---------------------------------------------------------------------- */

/* Per 256-vector of every weight row: fp32 FWHT with butterfly stages
 * h = 1, 2, ..., 128, then * 1/16; a = max|v|; s16 = fp16(f32(a/3));
 * q = clamp(rint(f32(v * f32(1/s16))), -3, 3) (all 0 if s16 == 0).
 * Storage (a layout of this library; the article fixes only 3-bit codes and
 * an fp16 scale per 256 weights): rows in blocks of 16, the last block
 * padded with zero rows (q = 0, s16 = 0); one 1568-byte record per (row
 * block, 256-chunk), records ordered [block][chunk], each holding the codes
 * c = q + 4 of the block's 16 rows:
 *   bytes    0..1023: 64 lanes x 16 bytes, lane l = 16 g + r (row r); byte m
 *                     holds bits 0-1 of codes 64 g + 16 t + m, t = 0..3, at
 *                     bits 2 t;
 *   bytes 1024..1535: 64 lanes x 8 bytes; byte 4 j + b holds bit 2 of code
 *                     64 g + 16 (u / 2) + 8 j + 4 (u % 2) + b at bit u;
 *   bytes 1536..1567: the 16 rows' fp16 scales.
 *   W       device, [d_out][d_in] fp32, d_in % 256 == 0.
 *   packed  device out, wush_had256_packed_bytes(d_out, d_in) bytes,
 *           16-byte aligned. */
size_t wush_had256_packed_bytes(int d_out, int d_in);
wush_status wush_had256_pack_weights(int d_out, int d_in, const float* W,
                                     uint8_t* packed, void* stream);

/* y[b][j] = sum_k x[b][k] * w_hat[j][k] with w_hat = s16 * (H_256 q) / 16 per
 * 256-vector (the inverse rotation of the dequantized codes).  Computed as
 * (s16/16) sum_m q_m (H_256 x)_m per vector (H_256 is symmetric), with the
 * rotated activations split into two int8 terms per 256-chunk (relative error
 * below 2^-15 of the chunk's largest value) and exact int32 dot products.
 *   x       device, [batch][d_in] bf16 bits, 16-byte aligned.
 *   packed  device, the output of wush_had256_pack_weights for (d_out, d_in).
 *   y       device out, [batch][d_out] fp32.
 *   ws      device scratch of at least wush_had256_gemv_ws_bytes(batch, d_in)
 *           bytes (16-byte aligned), or NULL (taken from the default memory
 *           pool per call, as for wush_w4a4_gemm); calls sharing a ws must be
 *           ordered on one stream.  Batches up to 4 need none (size 0):
 *           their activations are rotated and split inside the GEMV kernel.
 * Errors: WUSH_E_SHAPE (batch not in 1..16, d_in % 256, d_in > 2^24),
 * WUSH_E_ARG, WUSH_E_HIP. */
size_t wush_had256_gemv_ws_bytes(int batch, int d_in);
wush_status wush_had256_gemv(int batch, int d_out, int d_in, const uint16_t* x,
                             const uint8_t* packed, float* y, void* ws,
                             size_t ws_bytes, void* stream);

/* Unquantized rotation v = H_256 w / 16 per 256-vector, in place allowed
 * (in == out).  H/16 is orthogonal and its own inverse, so two calls return
 * the input exactly on integer data with |w| <= 2^15 ([ITQ3_S] round trip).
 *   in, out  device, [rows][d_in] fp32, d_in % 256 == 0. */
wush_status wush_had256_rotate(int rows, int d_in, const float* in, float* out, void* stream);

/* ------------------------------------------------------------------------ */
const char* wush_status_string(wush_status s);
const char* wush_last_error(void);
/* Library version string, e.g. "wush 0.1 gfx950". */
const char* wush_version(void);

#ifdef __cplusplus
}
#endif
#endif /* WUSH_H */
