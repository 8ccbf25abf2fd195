"""Pins for the oracle's transform-then-quantize step (CPU only)."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import fp, quant, transforms as tr, gemm
from synth.gen import random_case, CONFIGS, make_weights, make_activations

_libm = ctypes.CDLL("libm.so.6")
_c_fmaf = _libm.fmaf
_c_fmaf.restype = ctypes.c_float
_c_fmaf.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]


def test_apply_transform_matches_scalar_glibc_chain():
    """The vectorised chain equals a scalar loop of glibc fmaf calls."""
    W, X = random_case(1, 5, 64, 32)
    B = tr.activation_moments(X, 32).astype(np.float32)
    Tx, _, _, _ = tr.build_transforms("wush", W, B, 32)
    y = quant.apply_transform(Tx, X)
    for t in range(X.shape[0]):
        for b in range(2):
            for i in range(32):
                acc = 0.0
                for k in range(32):
                    acc = _c_fmaf(float(Tx[b, i, k]), float(X[t, 32 * b + k]), acc)
                assert np.float32(acc).view(np.uint32) == y[t, 32 * b + i].view(np.uint32)


def test_apply_transform_error_bound():
    """|y - T x| <= bs * u * sum|T||x| (fp32 dot-product bound), u = 2^-24."""
    W, X = random_case(2, 40, 128, 64)
    B = tr.activation_moments(X, 32).astype(np.float32)
    Tx, _, _, _ = tr.build_transforms("wush", W, B, 32)
    y = quant.apply_transform(Tx, X).astype(np.float64)
    Xb = X.astype(np.float64).reshape(40, 4, 32)
    T64 = Tx.astype(np.float64)
    exact = np.einsum("bik,tbk->tbi", T64, Xb).reshape(40, 128)
    bound = 32 * 2.0 ** -24 * np.einsum("bik,tbk->tbi", np.abs(T64), np.abs(Xb)).reshape(40, 128)
    assert np.all(np.abs(y - exact) <= bound * 1.0001)


def test_identity_is_bitwise_copy():
    _, X = random_case(3, 7, 64, 8)
    X[0, 0] = -0.0
    y = quant.apply_transform(None, X, identity=True)
    assert np.array_equal(y.view(np.uint32), X.view(np.uint32))


def _mx_brute(yblock):
    """Brute force MXFP4 of one 32-block: scale rule + per-element nearest code."""
    a = np.max(np.abs(yblock.astype(np.float64)))
    if a == 0:
        e = -127
    else:
        e = int(np.floor(np.log2(a))) - 2
        e = max(-127, min(127, e))
    codes = [fp.e2m1_code(np.float64(v) * 2.0 ** -e) for v in yblock]
    return e + 127, codes


def test_mxfp4_brute_force_and_scale_invariant():
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((20, 128)) * np.exp(rng.uniform(-10, 10, (20, 1)))).astype(np.float32)
    y[0, :32] = 0.0
    y[1, :32] = np.float32(2.0 ** -140)             # subnormal block: scale clamps at -127
    y[2, 5] = np.float32(6.0 * 2 ** 3)              # amax exactly on a power-of-two boundary
    codes, scales = quant.quant_mxfp4(y)
    c = quant.unpack_nibbles(codes)
    for r in range(20):
        for b in range(4):
            s, cc = _mx_brute(y[r, 32 * b:32 * b + 32])
            assert scales[r, b] == s
            assert list(c[r, 32 * b:32 * b + 32]) == [int(v) for v in cc]
            a = np.abs(y[r, 32 * b:32 * b + 32]).max()
            if a > 2.0 ** -120:
                assert 4.0 <= a * 2.0 ** -(int(s) - 127) < 8.0


def test_mxfp4_nan_block():
    y = np.ones((1, 64), np.float32)
    y[0, 40] = np.nan
    codes, scales = quant.quant_mxfp4(y)
    assert scales[0, 0] == 127 - 2                   # amax 1 -> e = -2
    assert scales[0, 1] == 255
    assert np.all(quant.unpack_nibbles(codes)[0, 32:] == 0)


def test_identity_mxfp4_is_plain_mxfp4():
    _, X = random_case(4, 16, 128, 8)
    c1, s1 = quant.transform_quant("mxfp4", None, X, identity=True)
    c2, s2 = quant.quant_mxfp4(X)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_nvfp4_scale_is_torch_e4m3_and_codes_nearest():
    rng = np.random.default_rng(6)
    y = (rng.standard_normal((16, 64)) * rng.uniform(0.01, 3, (16, 1))).astype(np.float32)
    g = quant.nvfp4_tensor_scale(y)
    codes, scales = quant.quant_nvfp4(y, g)
    yb = y.reshape(16, 4, 16)
    a = np.abs(yb).max(-1)
    s_raw = (a / np.float32(np.float32(6.0) * g)).astype(np.float32)
    ref = torch.from_numpy(np.minimum(s_raw, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref)
    c = quant.unpack_nibbles(codes).reshape(16, 4, 16)
    s_eff = (fp.e4m3_value(scales).astype(np.float32) * g).astype(np.float32)
    r = (np.float32(1) / s_eff).astype(np.float32)
    v = (yb * r[..., None]).astype(np.float32)
    dec = fp.e2m1_value(c)
    # nearest E2M1 magnitude with matching sign
    for val, code, dv in zip(v.ravel(), c.ravel(), dec.ravel()):
        mags = fp.E2M1_MAG
        assert abs(abs(val) - abs(dv)) == np.min(np.abs(abs(val) - mags))
        assert bool(code & 8) == bool(np.signbit(val))
    # decode error bounded by half a step of the coarsest level spacing
    assert np.all(np.abs(dec - v) <= 1.0 + 1e-12)


def test_int4_codes_are_nearest_level():
    rng = np.random.default_rng(7)
    y = (rng.standard_normal((10, 96)) * rng.uniform(0.01, 50, (10, 1))).astype(np.float32)
    codes, scales = quant.quant_int4(y)
    q = quant.unpack_nibbles(codes).astype(np.int64)
    q = np.where(q >= 8, q - 16, q).reshape(10, 3, 32)
    yb = y.reshape(10, 3, 32)
    a = np.abs(yb).max(-1)
    assert np.array_equal(scales, torch.from_numpy((a / np.float32(7)).astype(np.float32)).half().view(torch.int16).numpy().view(np.uint16))
    s = scales.view(np.float16).astype(np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    t = (yb * r[..., None]).astype(np.float64)
    levels = np.arange(-7, 8)
    for tv, qv in zip(t.ravel(), q.ravel()):
        d = np.abs(tv - levels)
        best = levels[d == d.min()]
        if len(best) == 2:                    # tie: even level
            best = best[best % 2 == 0]
        assert qv == best[0]


def test_int4_zero_block():
    y = np.zeros((2, 32), np.float32)
    codes, scales = quant.quant_int4(y)
    assert np.all(codes == 0) and np.all(scales == 0)


def test_tiny_workload_loss_ordering():
    """On outlier-heavy data the MXFP4 layer loss orders WUSH <= Hadamard <= identity."""
    w = CONFIGS["tiny"]
    W = make_weights(w)
    X = make_activations(w)
    B = tr.activation_moments(X, 32).astype(np.float32)
    Yref = gemm.reference_output(W, X)
    loss = {}
    for kind in ("identity", "hadamard", "wus", "wush"):
        Tx, Tw, _, _ = tr.build_transforms(kind, W, B, 32)
        ident = kind == "identity"
        ca, sa = quant.transform_quant("mxfp4", Tx, X, identity=ident)
        cw, sw = quant.transform_quant("mxfp4", Tw, W, identity=ident)
        Y = gemm.w4a4_gemm("mxfp4", ca, sa, cw, sw)
        loss[kind] = gemm.layer_loss(Y, Yref)
    assert loss["wush"] <= loss["hadamard"] <= loss["identity"], loss
    assert loss["wush"] < 0.5 * loss["identity"], loss


# ---------------------------------------------------------------------------
# Hadamard-diagonal transform (pinned fp32 butterflies)


@pytest.mark.parametrize("bs", [16, 32])
def test_apply_hd_matches_dense_product(bs):
    from oracle import transforms as tr
    rng = np.random.default_rng(40 + bs)
    x = rng.standard_normal((50, 4 * bs)).astype(np.float32)
    d = rng.uniform(0.05, 0.4, 4 * bs).astype(np.float32)
    y = quant.apply_hd(d, x, bs).astype(np.float64)
    T = tr.hd_dense(d, bs)                                    # H diag(d) per block
    ref = np.einsum("bij,nbj->nbi", T, x.astype(np.float64).reshape(50, 4, bs)).reshape(50, 4 * bs)
    # log2(bs) rounded stages after one rounded product
    tol = (np.log2(bs) + 1) * 2.0 ** -24 * np.abs(x * d).reshape(50, 4, bs).sum(-1, keepdims=True)
    assert np.all(np.abs(y - ref).reshape(50, 4, bs) <= tol)


def test_apply_hd_is_exact_on_integers_and_signs_follow_sylvester():
    import scipy.linalg
    rng = np.random.default_rng(44)
    x = rng.integers(-1000, 1001, (20, 64)).astype(np.float32)
    y = quant.apply_hd(np.ones(64, np.float32), x, 32)
    H = scipy.linalg.hadamard(32)
    ref = np.einsum("ij,nbj->nbi", H, x.astype(np.int64).reshape(20, 2, 32)).reshape(20, 64)
    assert np.array_equal(y.astype(np.int64), ref)
    # one-hot inputs read out the matrix columns, signs included
    e = np.zeros((32, 32), np.float32)
    np.fill_diagonal(e, 1.0)
    assert np.array_equal(quant.apply_hd(np.ones(32, np.float32), e, 32), H.T.astype(np.float32))


def test_transform_quant_hd_is_apply_then_quantize():
    rng = np.random.default_rng(45)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    d = rng.uniform(0.1, 0.3, 128).astype(np.float32)
    c1, s1 = quant.transform_quant_hd("mxfp4", d, x)
    c2, s2 = quant.quant_mxfp4(quant.apply_hd(d, x, 32))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


# ----------------------------------------------------------------------------- byte-layout pins
# Hand-derived bytes (tests/golden/packing.json): they do not go through the
# oracle's own unpack, so a swapped nibble order or a different NVFP4 tensor
# scale divisor fails here even though the matmul is invariant to both.

def _packing_golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "packing.json")) as f:
        return json.load(f)


def test_pack_nibbles_hand_rows():
    gold = _packing_golden()
    for row in gold["nibble_rows"]:
        got = quant.pack_nibbles(np.array([row["codes"]], np.uint8))
        assert list(got[0]) == row["bytes"]
        back = quant.unpack_nibbles(np.array([row["bytes"]], np.uint8))
        assert list(back[0]) == row["codes"]


def _block(spec, bs):
    y = np.full((1, bs), spec["rest"], np.float32)
    y[0, :len(spec["values_head"])] = spec["values_head"]
    return y


def test_mxfp4_block_hand_bytes():
    gold = _packing_golden()["mxfp4_block"]
    codes, scales = quant.quant_mxfp4(_block(gold, 32))
    assert int(scales[0, 0]) == gold["scale_byte"]
    head = gold["bytes_head"]
    assert list(codes[0, :len(head)]) == head
    assert np.all(codes[0, len(head):] == 0)


def test_int4_block_hand_bytes():
    gold = _packing_golden()["int4_block"]
    codes, scales = quant.quant_int4(_block(gold, 32))
    assert int(scales[0, 0]) == gold["scale_fp16_bits"]
    head = gold["bytes_head"]
    assert list(codes[0, :len(head)]) == head
    assert np.all(codes[0, len(head):] == 0)


def test_nvfp4_tensor_scale_hand_values():
    gold = _packing_golden()
    rng = np.random.default_rng(11)
    for case in gold["nvfp4_tensor_scale"]:
        y = rng.uniform(-1, 1, (8, 64)).astype(np.float32) * np.float32(case["amax"] / 2)
        y[3, 17] = -case["amax"]
        g = quant.nvfp4_tensor_scale(y)
        assert g.dtype == np.float32 and float(g) == case["g"]
        # the block that holds the tensor maximum takes the largest finite E4M3 scale
        _, scales = quant.quant_nvfp4(y, g)
        assert int(scales[3, 17 // 16]) == gold["nvfp4_max_block_scale_byte"]
        assert np.all(scales <= gold["nvfp4_max_block_scale_byte"])


def test_nvfp4_max_block_scale_at_any_amax():
    # for any tensor the block holding max|y| is scaled to 448 (byte 0x7E) and its
    # largest value encodes as the top E2M1 level, 6
    gold = _packing_golden()
    rng = np.random.default_rng(12)
    for _ in range(50):
        y = (rng.standard_normal((4, 48)) * np.exp(rng.uniform(-20, 20))).astype(np.float32)
        g = quant.nvfp4_tensor_scale(y)
        codes, scales = quant.quant_nvfp4(y, g)
        r, c = np.unravel_index(np.argmax(np.abs(y)), y.shape)
        assert int(scales[r, c // 16]) == gold["nvfp4_max_block_scale_byte"]
        assert int(quant.unpack_nibbles(codes)[r, c]) & 7 == 7
