"""Floating-point building blocks of the oracle (test infrastructure only).

* ``fmaf``           fp32 fused multiply-add with a single rounding (IEEE 754
                     fusedMultiplyAdd, round-to-nearest-even), elementwise.
* ``e2m1_code``      FP4 E2M1 encoder: nearest representable value, ties to
                     the even code, saturating at 6, sign copied.
* ``e2m1_value``     decoder of the 16 E2M1 codes.
* ``e8m0_*``         the power-of-two scale byte of MXFP4.
* ``e4m3_*``         FP8 E4M3 (finite-only "fn" variant) encoder / decoder.
* ``f16_bits``       fp16 round-to-nearest-even (numpy's cast) as raw bits.

The element formats are those named for the MXFP4 / NVFP4 / INT4 experiments
of the "WUSH" news article (paragraph on experiments).  The pages do not spell
the formats out; the definitions used here are the usual ones (OCP MX: 32
E2M1 values sharing one E8M0 exponent; NVFP4: 16 E2M1 values sharing one
E4M3 scale plus a per-tensor fp32 scale).
"""

import numpy as np

# ---------------------------------------------------------------------------
# fp32 FMA with one rounding
# ---------------------------------------------------------------------------


def fmaf(a, b, c):
    """Return fl32(a*b + c) with a single round-to-nearest-even.

    a, b, c are float32 arrays (broadcast).  Method: the product of two fp32
    values has at most 48 significant bits, so ``p = f64(a)*f64(b)`` is exact.
    ``s = p + c`` in fp64 is then correct up to one fp64 rounding whose error
    ``e`` TwoSum recovers exactly (p + c == s + e).  Rounding ``s`` to fp32
    gives the right answer except when ``s`` sits exactly on an fp32 rounding
    midpoint while ``e != 0``; then the exact value lies on the side of
    sign(e) and the result is the neighbour on that side.
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    c = np.asarray(c, dtype=np.float32)
    p = a.astype(np.float64) * b.astype(np.float64)
    c64 = c.astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        s = p + c64
        bv = s - p
        e = (p - (s - bv)) + (c64 - bv)
        r = s.astype(np.float32)
        r64 = r.astype(np.float64)
        inexact = (r64 != s) & np.isfinite(s) & np.isfinite(r64)
        if not np.any(inexact & (e != 0)):
            return r
        up = s > r64
        nb = np.where(up, np.nextafter(r, np.float32(np.inf)),
                      np.nextafter(r, np.float32(-np.inf)))
        mid = (r64 + nb.astype(np.float64)) * 0.5
        fix = inexact & (s == mid) & (e != 0)
        hi = np.maximum(r, nb)
        lo = np.minimum(r, nb)
        return np.where(fix, np.where(e > 0, hi, lo), r).astype(np.float32)


# ---------------------------------------------------------------------------
# FP4 E2M1
# ---------------------------------------------------------------------------

#: magnitudes of the 8 non-negative E2M1 codes (bit 3 is the sign)
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_code(v):
    """Encode values ``v`` (any float array) to 4-bit E2M1 codes (uint8).

    The magnitude code is the index of the nearest entry of E2M1_MAG; an exact
    tie between two neighbours goes to the even index (the code whose mantissa
    bit is 0).  Magnitudes beyond 6 saturate to 6 (index 7).  Bit 3 copies the
    sign bit of ``v``, including for -0 and for negative values that round to
    magnitude 0.  NaN encodes as 0.
    """
    v = np.asarray(v, dtype=np.float64)
    # every magnitude at or above 6 saturates to 6; clamping to 8 first keeps the
    # distances to the grid resolvable in fp64 for huge values and infinities
    mag = np.minimum(np.abs(v), 8.0)
    d = np.abs(mag[..., None] - E2M1_MAG)           # distance to every level
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin                                  # one or two nearest levels
    idx = np.arange(8)
    # among the nearest levels prefer an even index, then the smaller one
    key = np.where(cand, (idx % 2) * 16 + idx, 1000)
    code = key.argmin(axis=-1).astype(np.uint8)
    code = np.where(np.signbit(v), code | 8, code).astype(np.uint8)
    return np.where(np.isnan(v), 0, code).astype(np.uint8)


def e2m1_value(code):
    """Decode 4-bit E2M1 codes to float64 values."""
    code = np.asarray(code).astype(np.int64)
    mag = E2M1_MAG[code & 7]
    return np.where(code & 8, -mag, mag)


# ---------------------------------------------------------------------------
# E8M0 (power-of-two scale)
# ---------------------------------------------------------------------------


def e8m0_value(byte):
    """Decode an E8M0 scale byte: 2**(byte-127); 255 is NaN."""
    byte = np.asarray(byte).astype(np.int64)
    val = np.ldexp(1.0, byte - 127)
    return np.where(byte == 255, np.nan, val)


# ---------------------------------------------------------------------------
# FP8 E4M3 ("fn": no infinities, 0x7F / 0xFF are NaN, max 448)
# ---------------------------------------------------------------------------


def e4m3_value(byte):
    """Decode E4M3FN bytes to float64 (bias 7, subnormals m*2**-9)."""
    byte = np.asarray(byte).astype(np.int64)
    s = (byte >> 7) & 1
    ex = (byte >> 3) & 15
    m = byte & 7
    mag = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ex - 7))
    mag = np.where((ex == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


_E4M3_POS = e4m3_value(np.arange(0x7F))             # 0x00..0x7E, ascending


def e4m3_code(x):
    """Encode non-negative finite x <= 448 to E4M3FN, nearest, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    d = np.abs(x[..., None] - _E4M3_POS)
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin
    idx = np.arange(0x7F)
    key = np.where(cand, (idx % 2) * 1024 + idx, 1 << 20)
    return key.argmin(axis=-1).astype(np.uint8)


# ---------------------------------------------------------------------------
# fp16
# ---------------------------------------------------------------------------


def f16_bits(x):
    """fp16 round-to-nearest-even of float32 values, returned as uint16 bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_value(bits):
    """Decode fp16 bits to float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
