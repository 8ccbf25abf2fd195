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
* storage (this project's own layout; the page fixes only 3-bit codes with
  an fp16 scale per 256 weights): rows are grouped in blocks of 16 (the last
  block padded with rows of q = 0 and scale 0); each (row block, 256-chunk)
  is one 1568-byte record of the stored codes c = q + 4 in [1, 7]:
    - bytes [0, 1024): 64 lanes x 16 bytes, lane l = 16 g + r (row r of the
      block, code group g); byte m of lane l holds bits 0-1 of codes
      k = 64 g + 16 t + m, t = 0..3, at bits 2 t;
    - bytes [1024, 1536): 64 lanes x 8 bytes; byte 4 j + b of lane l holds
      bit 2 of code k = 64 g + 16 (u // 2) + 8 j + 4 (u % 2) + b at bit u,
      u = 0..7;
    - bytes [1536, 1568): the 16 rows' fp16 scales.
* decode: w_hat = f32(s16) * (H q) / 16, exact in fp64.
"""

import numpy as np

from .fp import f16_bits, f16_value
from .transforms import hadamard

VEC = 256


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


BLOCK_ROWS = 16
RECORD = 1568


def quantize(Wt):
    """Wt [d_out][d_in] fp32 -> (q [d_out][d_in/256][256] int64 in [-3, 3], s16 [d_out][d_in/256] fp16 bits)."""
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
    return q, s16


def _positions():
    """For code k of a chunk: its lane group g, low-plane byte m and bit 2t, high-plane byte and bit u."""
    k = np.arange(VEC)
    g, t, m = k // 64, (k % 64) // 16, k % 16
    i, b = m // 4, m % 4
    u, j = 2 * t + (i % 2), i // 2
    return g, m, 2 * t, 4 * j + b, u


def packed_bytes(d_out, d_in):
    return -(-d_out // BLOCK_ROWS) * (d_in // VEC) * RECORD


def pack_records(q, s16):
    """(q [d_out][nv][256], s16 [d_out][nv]) -> records [ceil(d_out/16)][nv][1568] uint8."""
    d_out, nv, _ = q.shape
    nrb = -(-d_out // BLOCK_ROWS)
    c = np.full((nrb * BLOCK_ROWS, nv, VEC), 4, dtype=np.int64)
    c[:d_out] = q + 4
    s = np.zeros((nrb * BLOCK_ROWS, nv), dtype=np.uint16)
    s[:d_out] = s16
    c = c.reshape(nrb, BLOCK_ROWS, nv, VEC).transpose(0, 2, 1, 3)          # [rb][v][r][k]
    s = s.reshape(nrb, BLOCK_ROWS, nv).transpose(0, 2, 1)                  # [rb][v][r]
    rec = np.zeros((nrb, nv, RECORD), dtype=np.uint8)
    g, m, sh, hb, u = _positions()
    for r in range(BLOCK_ROWS):
        lane = 16 * g + r
        for k in range(VEC):
            rec[:, :, 16 * lane[k] + m[k]] |= ((c[:, :, r, k] & 3) << sh[k]).astype(np.uint8)
            rec[:, :, 1024 + 8 * lane[k] + hb[k]] |= (((c[:, :, r, k] >> 2) & 1) << u[k]).astype(np.uint8)
    rec[:, :, 1536:] = np.ascontiguousarray(s.astype("<u2")).view(np.uint8).reshape(nrb, nv, 2 * BLOCK_ROWS)
    return rec


def unpack_records(rec, d_out):
    """records -> (q [d_out][nv][256] int64, s16 [d_out][nv] uint16)."""
    rec = np.asarray(rec, dtype=np.uint8)
    nrb, nv, _ = rec.shape
    g, m, sh, hb, u = _positions()
    q = np.zeros((nrb, nv, BLOCK_ROWS, VEC), dtype=np.int64)
    for r in range(BLOCK_ROWS):
        lane = 16 * g + r
        lo = (rec[:, :, 16 * lane + m] >> sh) & 3
        hi = (rec[:, :, 1024 + 8 * lane + hb] >> u) & 1
        q[:, :, r, :] = (lo | (hi << 2)).astype(np.int64) - 4
    s = np.ascontiguousarray(rec[:, :, 1536:]).view("<u2").reshape(nrb, nv, BLOCK_ROWS)
    q = q.transpose(0, 2, 1, 3).reshape(nrb * BLOCK_ROWS, nv, VEC)[:d_out]
    s = s.transpose(0, 2, 1).reshape(nrb * BLOCK_ROWS, nv)[:d_out].astype(np.uint16)
    return q, s


def pack_weights(Wt):
    """Wt [d_out][d_in] fp32 -> records [ceil(d_out/16)][d_in/256][1568] uint8."""
    return pack_records(*quantize(Wt))


def decode_weights(rec, d_out):
    """Exact fp64 w_hat [d_out][d_in] = s * (H q) / 16 per 256-vector."""
    q, s16 = unpack_records(rec, d_out)
    H = hadamard(VEC)
    hq = q.astype(np.float64) @ H.T                     # H symmetric
    w = hq * f16_value(s16)[..., None] / 16.0
    return w.reshape(w.shape[0], -1)


def gemv(x, rec, d_out):
    """y [B][d_out] = x [B][d_in] @ w_hat^T in fp64."""
    return np.asarray(x, dtype=np.float64) @ decode_weights(rec, d_out).T
