"""Pins for the oracle's floating-point building blocks (CPU only)."""

import ctypes
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

_libm = ctypes.CDLL("libm.so.6")
_c_fmaf = _libm.fmaf
_c_fmaf.restype = ctypes.c_float
_c_fmaf.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]


def _rand_f32(rng, n, emin=-30, emax=30):
    m = rng.uniform(1.0, 2.0, size=n)
    e = rng.integers(emin, emax, size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    return (s * np.ldexp(m, e)).astype(np.float32)


def _frac_fmaf(a, b, c):
    """Correctly rounded fp32 of a*b+c computed with exact rationals (ties to even)."""
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    r = np.float32(float(exact))                     # may be off by double rounding
    cands = [np.nextafter(r, np.float32(-np.inf)), r, np.nextafter(r, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact),
                                     int(np.array(v, np.float32).view(np.uint32)) & 1))
    if exact == 0:
        return np.float32(float(a) * float(b) + float(c))
    return np.float32(best)


def _midpoint_cases():
    # exact results just above / below an fp32 midpoint that fp64 rounds onto it
    a = np.float32(1 - 2.0 ** -15)
    b = np.float32(1 + 2.0 ** -15)          # a*b = 1 - 2^-30
    cases = []
    for c in (2.0 ** 24, 2.0 ** 24 + 2, 2.0 ** 25 + 4, 3 * 2.0 ** 23):
        for sa in (1.0, -1.0):
            cases.append((np.float32(sa) * a, b, np.float32(c)))
            cases.append((np.float32(sa) * a, b, np.float32(-c)))
    return cases


def test_fmaf_matches_glibc_random():
    rng = np.random.default_rng(0)
    n = 20000
    a = _rand_f32(rng, n)
    b = _rand_f32(rng, n)
    c = (a.astype(np.float64) * b.astype(np.float64) * rng.uniform(-2, 2, n)).astype(np.float32)
    c[::3] = _rand_f32(rng, len(c[::3]))
    got = fp.fmaf(a, b, c)
    ref = np.array([_c_fmaf(float(x), float(y), float(z)) for x, y, z in zip(a, b, c)],
                   dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_fmaf_midpoints_vs_glibc_and_fractions():
    cases = _midpoint_cases()
    a, b, c = (np.array(v, dtype=np.float32) for v in zip(*cases))
    got = fp.fmaf(a, b, c)
    for i, (x, y, z) in enumerate(cases):
        g = np.float32(_c_fmaf(float(x), float(y), float(z)))
        f = _frac_fmaf(x, y, z)
        assert got[i].view(np.uint32) == g.view(np.uint32), (x, y, z)
        assert got[i].view(np.uint32) == f.view(np.uint32), (x, y, z)
    # the fix-up is actually exercised: plain fp64-then-fp32 double-rounds one of them
    naive = (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)
    assert not np.array_equal(naive.view(np.uint32), got.view(np.uint32))


def test_fmaf_subnormal_and_zero_signs():
    rng = np.random.default_rng(1)
    a = _rand_f32(rng, 4000, -140, -60)
    b = _rand_f32(rng, 4000, -20, 10)
    c = _rand_f32(rng, 4000, -150, -100)
    a[:10] = 0.0
    b[10:20] = -0.0
    c[:30] = -0.0
    got = fp.fmaf(a, b, c)
    ref = np.array([_c_fmaf(float(x), float(y), float(z)) for x, y, z in zip(a, b, c)],
                   dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_fmaf_fraction_spot_check():
    rng = np.random.default_rng(2)
    a = _rand_f32(rng, 300)
    b = _rand_f32(rng, 300)
    c = (-a.astype(np.float64) * b.astype(np.float64) * (1 + rng.uniform(-1e-6, 1e-6, 300))).astype(np.float32)
    got = fp.fmaf(a, b, c)
    for i in range(300):
        assert got[i].view(np.uint32) == _frac_fmaf(a[i], b[i], c[i]).view(np.uint32)


# --------------------------------------------------------------------------- E2M1


def _e2m1_threshold(v):
    """Independent E2M1 encoder: count the rounding thresholds a magnitude passes."""
    m = abs(v)
    code = int(m > 0.25) + int(m >= 0.75) + int(m > 1.25) + int(m >= 1.75) \
        + int(m > 2.5) + int(m >= 3.5) + int(m > 5.0)
    if np.isnan(v):
        return 0
    return code | (8 if np.signbit(v) else 0)


def test_e2m1_golden_ties():
    with open(os.path.join(GOLDEN, "e2m1_ties.json")) as f:
        g = json.load(f)
    for v, code in g["cases"]:
        assert int(fp.e2m1_code(np.float64(float(v)))) == code, v


def test_e2m1_against_thresholds_and_brute_force():
    rng = np.random.default_rng(3)
    grid = np.concatenate([np.arange(-8, 8.0001, 0.125), [-0.0, 0.0, np.nan, 1e9, -1e9, 1e-30, -1e-30],
                           [1e20, -1e20, 3.4e38, np.inf, -np.inf]])
    vals = np.concatenate([grid, rng.uniform(-9, 9, 5000)])
    codes = fp.e2m1_code(vals)
    dec = fp.e2m1_value(np.arange(16))
    for v, c in zip(vals, codes):
        assert c == _e2m1_threshold(v), v
        if np.isnan(v):
            continue
        # brute force over all 16 codes: nearest value with the sign of v
        d = np.abs(min(abs(v), 8.0) * np.sign(v) - dec) if np.isfinite(v) or np.isinf(v) else np.abs(v - dec)
        same_sign = np.array([np.signbit(v) == bool(k & 8) for k in range(16)])
        d = np.where(same_sign, d, np.inf)
        assert d[c] == d.min()


def test_e2m1_value_table():
    # the 8 magnitudes are sign x 2^(e-1) x (1 + m/2) for e>0, and m/2 for e==0
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m * 0.5) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert fp.e2m1_value(code) == (-mag if s else mag)


# --------------------------------------------------------------------------- E8M0 / E4M3 / fp16


def test_e8m0_values():
    assert fp.e8m0_value(127) == 1.0
    assert fp.e8m0_value(0) == 2.0 ** -127
    assert fp.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(fp.e8m0_value(255))


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(4)
    x = np.concatenate([
        rng.uniform(0, 448, 20000), np.exp(rng.uniform(np.log(1e-4), np.log(448), 20000)),
        fp.e4m3_value(np.arange(0x7F)),                          # exact grid points
        (fp.e4m3_value(np.arange(0x7E)) + fp.e4m3_value(np.arange(1, 0x7F))) / 2,  # ties
        [0.0, 2.0 ** -10, 2.0 ** -10 * 1.0001, 448.0],
    ]).astype(np.float32)
    ours = fp.e4m3_code(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    assert np.allclose(fp.e4m3_value(ours), torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy())


def test_f16_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10, np.exp(rng.uniform(-20, 11, 20000)),
                        [1 / 3, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 65504.0, 65520.0]]).astype(np.float32)
    ours = fp.f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert fp.f16_bits(np.float32(1 / 3)) == 0x3555
