"""Pins for the oracle's quantized GEMM, layer loss and Hadamard-256 path (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import fp, quant, gemm, had256
from synth.gen import random_case


def _frac_decode_mx(codes, scales):
    c = quant.unpack_nibbles(codes)
    rows, K = c.shape
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            code = int(c[r, k])
            mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
                   Fraction(3), Fraction(4), Fraction(6)][code & 7]
            v = -mag if code & 8 else mag
            e = int(scales[r, k // 32]) - 127
            row.append(v * (Fraction(2) ** e))
        out.append(row)
    return out


def test_mxfp4_gemm_exact_on_tiny():
    W, X = random_case(5, 6, 64, 5)
    ca, sa = quant.quant_mxfp4(X)
    cw, sw = quant.quant_mxfp4(W)
    Y = gemm.w4a4_gemm("mxfp4", ca, sa, cw, sw)
    A = _frac_decode_mx(ca, sa)
    B = _frac_decode_mx(cw, sw)
    for m in range(6):
        for n in range(5):
            exact = sum(a * b for a, b in zip(A[m], B[n]))
            assert Fraction(Y[m, n]) == exact          # fp64 holds it exactly here


def test_nvfp4_and_int4_decode_brute_force():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((3, 64)).astype(np.float32)
    g = quant.nvfp4_tensor_scale(y)
    c, s = quant.quant_nvfp4(y, g)
    d = gemm.decode("nvfp4", c, s, g)
    cu = quant.unpack_nibbles(c)
    for r in range(3):
        for k in range(64):
            assert d[r, k] == fp.e2m1_value(cu[r, k]) * fp.e4m3_value(s[r, k // 16]) * float(g)
    c, s = quant.quant_int4(y)
    d = gemm.decode("int4", c, s)
    cu = quant.unpack_nibbles(c).astype(int)
    for r in range(3):
        for k in range(64):
            q = cu[r, k] - 16 if cu[r, k] >= 8 else cu[r, k]
            assert d[r, k] == q * float(np.uint16(s[r, k // 32]).view(np.float16))


def test_quantization_error_small_relative_to_signal():
    W, X = random_case(6, 64, 256, 48, outliers=0)
    for fmt in ("mxfp4", "nvfp4", "int4"):
        g = quant.nvfp4_tensor_scale(X) if fmt == "nvfp4" else None
        dx = gemm.decode(fmt, *quant.transform_quant(fmt, None, X, g=g, identity=True), g)
        rel = np.linalg.norm(dx - X) / np.linalg.norm(X)
        assert 0.02 < rel < 0.2, (fmt, rel)          # a 4-bit grid: a few percent


def test_layer_loss_definition():
    rng = np.random.default_rng(9)
    Y = rng.standard_normal((7, 11))
    R = Y + 0.5
    assert gemm.layer_loss(Y, R) == pytest.approx(0.25, rel=1e-15)
    assert gemm.layer_loss(R, R) == 0.0


# --------------------------------------------------------------------------- Hadamard-256


def test_fwht_equals_dense_hadamard():
    rng = np.random.default_rng(10)
    v = rng.standard_normal((20, 256)).astype(np.float32)
    got = had256.fwht256(v).astype(np.float64)
    H = scipy.linalg.hadamard(256).astype(np.float64)
    ref = v.astype(np.float64) @ H.T / 16
    bound = 8 * 2.0 ** -24 * (np.abs(v).astype(np.float64) @ np.abs(H).T) / 16
    assert np.all(np.abs(got - ref) <= bound)
    ints = rng.integers(-2 ** 15, 2 ** 15, (20, 256)).astype(np.float32)
    assert np.array_equal(had256.fwht256(ints).astype(np.float64), ints.astype(np.float64) @ H.T / 16)


def test_fwht_round_trip():
    rng = np.random.default_rng(11)
    ints = rng.integers(-2 ** 15, 2 ** 15 + 1, (50, 256)).astype(np.float32)
    assert np.array_equal(had256.fwht256(had256.fwht256(ints)), ints)   # exact
    v = rng.standard_normal((50, 256)).astype(np.float32)
    rt = had256.fwht256(had256.fwht256(v))
    assert np.all(np.abs(rt - v) <= 16 * 2.0 ** -24 * np.abs(v).max(axis=1, keepdims=True))


def test_had256_codes_nearest_and_record_layout():
    W, _ = random_case(12, 1, 512, 6)
    q, s16 = had256.quantize(W)
    assert q.shape == (6, 2, 256) and s16.shape == (6, 2)
    v = had256.fwht256(W.reshape(6, 2, 256))
    s = s16.view(np.float16).astype(np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    t = (v * r[..., None]).astype(np.float64)
    lv = np.arange(-3, 4)
    for tv, qv in zip(t.ravel(), q.ravel()):
        d = np.abs(tv - lv)
        best = lv[d == d.min()]
        if len(best) == 2:
            best = best[best % 2 == 0]
        assert qv == best[0]
    # record layout, checked bit by bit from its definition; 6 rows -> one
    # block with 10 padding rows of q = 0 (stored 4) and scale 0
    rec = had256.pack_weights(W)
    assert rec.shape == (1, 2, 1568) and had256.packed_bytes(6, 512) == rec.size
    for vv in range(2):
        for row in range(16):
            for k in range(256):
                c = q[row, vv, k] + 4 if row < 6 else 4
                g, rest = divmod(k, 64)
                t, m = divmod(rest, 16)
                lane = 16 * g + row
                assert (rec[0, vv, 16 * lane + m] >> (2 * t)) & 3 == c & 3
                i, b = divmod(m, 4)
                u = 2 * t + i % 2
                assert (rec[0, vv, 1024 + 8 * lane + 4 * (i // 2) + b] >> u) & 1 == c >> 2
            sc = int(rec[0, vv, 1536 + 2 * row]) | (int(rec[0, vv, 1537 + 2 * row]) << 8)
            assert sc == (int(s16[row, vv]) if row < 6 else 0)
    q2, s2 = had256.unpack_records(rec, 6)
    assert np.array_equal(q2, q) and np.array_equal(s2, s16)


def test_had256_gemv_matches_decoded_product():
    W, _ = random_case(13, 1, 512, 8)
    rec = had256.pack_weights(W)
    x = np.random.default_rng(14).standard_normal((3, 512))
    y = had256.gemv(x, rec, 8)
    w = had256.decode_weights(rec, 8)
    # decoded weights approximate W (3-bit after rotation)
    assert np.linalg.norm(w - W) / np.linalg.norm(W) < 0.35
    assert np.allclose(y, x @ w.T, rtol=1e-12)
    # the decode is the inverse rotation of s*q: check against the fp32 FWHT on integers
    q, s16 = had256.unpack_records(rec, 8)
    inv = had256.fwht256(q.astype(np.float32)).astype(np.float64) * s16.view(np.float16).astype(np.float64)[..., None]
    assert np.array_equal(inv.reshape(8, 512), w)
