"""256-point Walsh-Hadamard pre-rotation with 3-bit weight codes (test infrastructure only).

Source: "ITQ3_S" article (ai.866data.com), section on the core technique:
every 256-element weight vector is rotated by a fast Walsh-Hadamard transform
before a uniform 3-bit quantizer; the inverse transform is applied when the
weights are loaded for the matmul, and the rotate / inverse-rotate round trip
is exact.  The page's word for the code set reads as "ternary" but it speaks
of 3-bit quantization; the reading used is symmetric 3-bit levels [-3, 3].

Pinned arithmetic:
* forward FWHT in fp32, in place, stages h = 1, 2, 4, ..., 128; in each stage
  every pair (j, j + h) with j in a 2h-aligned group's lower half becomes
  (v[j] + v[j+h], v[j] - v[j+h]); then v *= 1/16 (exact).  H/16 is orthogonal
  and its own inverse.
* a = max|v|; s16 = fp16(f32(a / 3)); r = f32(1 / f32(s16)) (s16 == 0 -> codes 0);
  q = clamp(rint_even(f32(v r)), -3, 3).
* storage per 256-vector: 96 bytes = 64 bytes of bits 0-1 (code k in byte
  k // 4 at bit 2 (k % 4)) followed by 32 bytes of bit 2 (code k in byte
  64 + k // 8 at bit k % 8), codes being q & 7; one fp16 scale.
* decode: w_hat = f32(s16) * (H q) / 16, exact in fp64.
"""

import numpy as np

from .fp import f16_bits, f16_value
from .transforms import hadamard

VEC = 256
BYTES = 96


def fwht256(v):
    """Forward FWHT (unnormalised butterflies, then * 1/16) in fp32 over the last axis."""
    v = np.array(v, dtype=np.float32, copy=True)
    shp = v.shape
    v = v.reshape(-1, VEC)
    h = 1
    while h < VEC:
        w = v.reshape(v.shape[0], VEC // (2 * h), 2, h)
        lo = w[:, :, 0, :].copy()
        hi = w[:, :, 1, :].copy()
        w[:, :, 0, :] = lo + hi
        w[:, :, 1, :] = lo - hi
        v = w.reshape(-1, VEC)
        h *= 2
    v = (v * np.float32(0.0625)).astype(np.float32)
    return v.reshape(shp)


def pack_weights(Wt):
    """Wt [d_out][d_in] fp32 -> (planes [d_out][d_in/256][96] u8, scales [d_out][d_in/256] u16)."""
    Wt = np.asarray(Wt, dtype=np.float32)
    d_out, d_in = Wt.shape
    nv = d_in // VEC
    v = fwht256(Wt.reshape(d_out, nv, VEC))
    a = np.max(np.abs(v), axis=-1)
    s16 = f16_bits((a / np.float32(3.0)).astype(np.float32))
    s32 = s16.view(np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (np.float32(1.0) / s32).astype(np.float32)
        t = (v * r[..., None]).astype(np.float32)
    q = np.clip(np.rint(np.where(np.isfinite(t), t, 0.0)), -3, 3).astype(np.int64)
    q = np.where((s32 == 0)[..., None], 0, q)
    c = (q & 7).astype(np.uint8)                       # [o][v][256]
    planes = np.zeros((d_out, nv, BYTES), dtype=np.uint8)
    lo2 = c & 3
    for k in range(VEC):
        planes[:, :, k // 4] |= (lo2[:, :, k] << (2 * (k % 4))).astype(np.uint8)
        planes[:, :, 64 + k // 8] |= (((c[:, :, k] >> 2) & 1) << (k % 8)).astype(np.uint8)
    return planes, s16


def unpack_codes(planes):
    """planes [..][96] -> signed codes q [..][256] (int64)."""
    planes = np.asarray(planes, dtype=np.uint8)
    k = np.arange(VEC)
    lo2 = (planes[..., k // 4] >> (2 * (k % 4))) & 3
    b2 = (planes[..., 64 + k // 8] >> (k % 8)) & 1
    c = (lo2 | (b2 << 2)).astype(np.int64)
    return np.where(c >= 4, c - 8, c)


def decode_weights(planes, scales):
    """Exact fp64 w_hat [d_out][d_in] = s * (H q) / 16 per 256-vector."""
    q = unpack_codes(planes).astype(np.float64)        # [o][v][256]
    H = hadamard(VEC)
    hq = q @ H.T                                        # H symmetric
    w = hq * f16_value(scales)[..., None] / 16.0
    return w.reshape(w.shape[0], -1)


def gemv(x, planes, scales):
    """y [B][d_out] = x [B][d_in] @ w_hat^T in fp64."""
    return np.asarray(x, dtype=np.float64) @ decode_weights(planes, scales).T
