"""Full-size GPU parity on the five evaluation workloads (sampled outputs).

Each test runs the library at the workload's real shape, in the launch
configuration bench.py times, and compares outputs the oracle can compute one
by one: codes and scales of sampled token rows and weight rows bit-exactly,
and matmul outputs Y[sampled tokens][sampled columns] within the per-element
tolerance 1e-3 * max(|ref|, rms(ref)).  The oracle builds its own transforms
and codes from the seeded inputs.  The NVFP4 activation tensor scale is an
input of the call (a calibration value); the tests pass the oracle's value
computed on a calibration subset of tokens.
"""

import numpy as np
import pytest
import torch

import aware_block_transforms_amd as W
from oracle import quant, transforms as tr, gemm as og, had256 as oh
from synth.gen import CONFIGS, make_weights, make_activations, bf16_bits, bf16_round
from gpu_util import DEV, to_dev, x_dev, host, scales_np, gemm_close

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))
    return idx


def _layer_check(wl, fmt, kind, Wt, X, n_tok=48, n_w=48, seed=0):
    bs = W.BLOCK[fmt]
    ident = kind == "identity"
    n, d_in = X.shape
    d_out = Wt.shape[0]
    print(f"[fullsize] {wl.name} {fmt} {kind} n={n} d_in={d_in} d_out={d_out}", flush=True)
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    hd = kind == "hd"          # the Hadamard-diagonal variant: per-channel scales
    if hd:
        Tx, Tw, _, _ = tr.build_hd(Wt, Sx, bs)

        def apply(T, rows):
            return quant.apply_hd(T, rows, bs)

        def tq(T, rows, g):
            return quant.transform_quant_hd(fmt, T, rows, g=g)
    else:
        Tx, Tw, _, _ = tr.build_transforms(kind, Wt, Sx, bs)

        def apply(T, rows):
            return quant.apply_transform(T, rows, identity=ident)

        def tq(T, rows, g):
            return quant.transform_quant(fmt, T, rows, g=g, identity=ident)
    tok = _sample(n, n_tok, seed)
    wrow = _sample(d_out, n_w, seed + 1)
    # NVFP4 scales: activations from a calibration subset (an input), weights over all rows
    g_x = g_w = None
    if fmt == "nvfp4":
        cal = _sample(n, 256, seed + 2)
        g_x = quant.nvfp4_tensor_scale(apply(Tx, X[cal]))
        g_w = quant.nvfp4_tensor_scale(apply(Tw, Wt))

    # device: the same calls bench.py times
    sdt = torch.int16 if fmt == "int4" else torch.uint8
    xc = torch.empty((n, d_in // 2), dtype=torch.uint8, device=DEV)
    xs = torch.empty((n, d_in // bs), dtype=sdt, device=DEV)
    wc = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=DEV)
    wsc = torch.empty((d_out, d_in // bs), dtype=sdt, device=DEV)
    if hd:
        W.wush_transform_quant_hd(fmt, x_dev(X, wl.dtype), to_dev(Tx), xc, xs, g=g_x or 0.0)
        gw_dev = W.wush_pack_weights_hd(fmt, to_dev(Wt), to_dev(Tw), wc, wsc)
    else:
        W.wush_transform_quant(fmt, x_dev(X, wl.dtype), None if ident else to_dev(Tx), xc, xs, g=g_x or 0.0)
        gw_dev = W.wush_pack_weights(fmt, to_dev(Wt), None if ident else to_dev(Tw), wc, wsc)
    Y = torch.empty((n, d_out), dtype=torch.float32, device=DEV)
    W.wush_w4a4_gemm(fmt, xc, xs, wc, wsc, Y, a_g=g_x or 1.0, b_g=gw_dev)
    torch.cuda.synchronize()
    if fmt == "mxfp4" and not hd and kind != "identity" and d_in % 256 == 0:
        # the plane-ordered scale path bench.py times: the same codes and a bit-identical Y
        xc2 = torch.empty_like(xc)
        pa = torch.empty(W.wush_mxfp4_planes_bytes(n, d_in), dtype=torch.uint8, device=DEV)
        pb = torch.empty(W.wush_mxfp4_planes_bytes(d_out, d_in), dtype=torch.uint8, device=DEV)
        W.wush_transform_quant_mx_planes(x_dev(X, wl.dtype), to_dev(Tx), xc2, pa)
        W.wush_mxfp4_scale_planes(wsc, pb, d_in)
        Y2 = torch.empty_like(Y)
        W.wush_w4a4_gemm_mx_planes(xc2, pa, wc, pb, Y2)
        torch.cuda.synchronize()
        assert torch.equal(xc2, xc)
        assert torch.equal(Y2.view(torch.int32), Y.view(torch.int32))
        del xc2, pa, pb, Y2

    # oracle on the sampled rows
    rc, rs = tq(Tx, X[tok], g_x)
    assert np.array_equal(scales_np(xs, fmt)[tok], rs)
    assert np.array_equal(host(xc)[tok], rc)
    wrc, wrs = tq(Tw, Wt[wrow], g_w)
    assert np.array_equal(scales_np(wsc, fmt)[wrow], wrs)
    assert np.array_equal(host(wc)[wrow], wrc)
    if fmt == "nvfp4":
        assert np.float32(gw_dev) == g_w
    ref = og.w4a4_gemm(fmt, rc, rs, wrc, wrs, g_x, g_w)
    Ys = host(Y)[np.ix_(tok, wrow)]
    ok, worst = gemm_close(Ys, ref)
    assert ok, (wl.name, fmt, kind, worst)
    return Y


def test_fullsize_tiny_layer_with_loss():
    wl = CONFIGS["tiny"]
    Wt, X = make_weights(wl), make_activations(wl)
    for kind in wl.kinds:
        Y = _layer_check(wl, "mxfp4", kind, Wt, X, n_tok=200, n_w=300)
        # whole-output loss against the exact product
        bs = 32
        Sx = tr.activation_moments(X, bs).astype(np.float32)
        Tx, Tw, _, _ = tr.build_transforms(kind, Wt, Sx, bs)
        ident = kind == "identity"
        ca, sa = quant.transform_quant("mxfp4", Tx, X, identity=ident)
        cw, sw = quant.transform_quant("mxfp4", Tw, Wt, identity=ident)
        Yref = og.reference_output(Wt, X)
        l_ref = og.layer_loss(og.w4a4_gemm("mxfp4", ca, sa, cw, sw), Yref)
        ws = torch.empty(W.wush_loss_ws_bytes(*Y.shape) // 8, dtype=torch.float64, device=DEV)
        out = torch.empty(1, dtype=torch.float64, device=DEV)
        W.wush_layer_loss(Y, to_dev(Yref.astype(np.float32)), out, ws)
        torch.cuda.synchronize()
        assert abs(out.item() - l_ref) <= 1e-3 * l_ref, (kind, out.item(), l_ref)


def test_fullsize_qwen3_8b_up():
    wl = CONFIGS["qwen3_8b_up"]
    _layer_check(wl, "mxfp4", "wush", make_weights(wl), make_activations(wl))


def test_fullsize_qwen3_8b_up_hd():
    wl = CONFIGS["qwen3_8b_up"]
    _layer_check(wl, "mxfp4", "hd", make_weights(wl), make_activations(wl))


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_fullsize_square_sweep_hd(fmt):
    wl = CONFIGS["square_sweep"]
    _layer_check(wl, fmt, "hd", make_weights(wl), make_activations(wl), n_tok=24, n_w=24)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_fullsize_square_sweep(fmt):
    wl = CONFIGS["square_sweep"]
    Wt, X = make_weights(wl), make_activations(wl)
    for kind in wl.kinds:
        _layer_check(wl, fmt, kind, Wt, X, n_tok=24, n_w=24)


@pytest.mark.parametrize("which", ["qwen3_14b_up", "qwen3_14b_down"])
def test_fullsize_qwen3_14b(which):
    wl = CONFIGS[which]
    _layer_check(wl, "mxfp4", "wush", make_weights(wl), make_activations(wl), n_tok=32, n_w=32)


def test_fullsize_had256():
    wl = CONFIGS["had256"]
    Wt = make_weights(wl)
    d_out, d_in = Wt.shape
    print(f"[fullsize] {wl.name} d_in={d_in} d_out={d_out}", flush=True)
    nv, nrb = d_in // 256, d_out // 16
    packed = torch.empty((W.wush_had256_packed_bytes(d_out, d_in),), dtype=torch.uint8, device=DEV)
    W.wush_had256_pack_weights(to_dev(Wt), packed)
    torch.cuda.synchronize()
    blocks = _sample(nrb, 6, 5)                       # 16-row blocks, first and last included
    rows = (16 * blocks[:, None] + np.arange(16)).ravel()
    rp = oh.pack_weights(Wt[rows])
    assert np.array_equal(host(packed).reshape(nrb, nv, 1568)[blocks], rp)
    rng = np.random.default_rng([5, 1])
    for B in wl.extra["batches"]:
        x = make_activations(wl, n=B)
        y = torch.full((B, d_out), np.nan, dtype=torch.float32, device=DEV)
        W.wush_had256_gemv(to_dev(bf16_bits(x).view(np.int16)), packed, y)
        torch.cuda.synchronize()
        ref = oh.gemv(x, rp, len(rows))
        ok, worst = gemm_close(host(y)[:, rows], ref)
        assert ok, (B, worst)
    # round trip of the unquantized rotation on integer data at full width
    ints = rng.integers(-2 ** 15, 2 ** 15 + 1, (64, d_in)).astype(np.float32)
    a = to_dev(ints)
    W.wush_had256_rotate(a, a)
    W.wush_had256_rotate(a, a)
    torch.cuda.synchronize()
    assert np.array_equal(host(a), ints)


def test_fullsize_had256_outlier_activations():
    # Activations with outlier channels (x50 on 0.1% of the 4096 channels, plus
    # one channel at x1000): the GEMV rotates and splits the activations per
    # 256-chunk into two int8 terms, whose rounding error grows with the chunk
    # maximum, so the criterion is checked where the maximum is largest.
    wl = CONFIGS["had256"]
    Wt = make_weights(wl)
    d_out, d_in = Wt.shape
    print(f"[fullsize] {wl.name} outlier activations d_in={d_in} d_out={d_out}", flush=True)
    nv, nrb = d_in // 256, d_out // 16
    packed = torch.empty((W.wush_had256_packed_bytes(d_out, d_in),), dtype=torch.uint8, device=DEV)
    W.wush_had256_pack_weights(to_dev(Wt), packed)
    torch.cuda.synchronize()
    blocks = _sample(nrb, 6, 7)
    rows = (16 * blocks[:, None] + np.arange(16)).ravel()
    rp = oh.pack_weights(Wt[rows])
    rng = np.random.default_rng([5, 9])
    ch = rng.choice(d_in, 5, replace=False)
    for B in wl.extra["batches"]:
        x = make_activations(wl, n=B)
        x[:, ch[:4]] *= 50.0
        x[:, ch[4]] *= 1000.0
        x = bf16_round(x)
        y = torch.full((B, d_out), np.nan, dtype=torch.float32, device=DEV)
        W.wush_had256_gemv(to_dev(bf16_bits(x).view(np.int16)), packed, y)
        torch.cuda.synchronize()
        ref = oh.gemv(x, rp, len(rows))
        ok, worst = gemm_close(host(y)[:, rows], ref)
        assert ok, (B, worst)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_fullsize_streamed_x_each_format(fmt):
    # x larger than the 256 MB Infinity Cache takes the kernels whose x loads are
    # non-temporal (fp32 x of 2080 x 32768 = 272.6 MB, an even count of 32-blocks
    # and a multiple of four 16-blocks, so the merged-store kernels); codes and
    # scales of sampled tokens bit-exact against the oracle.  The transforms are
    # seeded random matrices: the kernel takes T as given.
    bs = W.BLOCK[fmt]
    n, d_in = 2080, 32768
    assert n * d_in * 4 > 256 << 20
    print(f"[fullsize] streamed x {fmt} n={n} d_in={d_in}", flush=True)
    rng = np.random.default_rng([11, bs])
    X = rng.standard_normal((n, d_in), dtype=np.float32)
    X[:, rng.choice(d_in, 32, replace=False)] *= 40
    T = (rng.standard_normal((d_in // bs, bs, bs)) / np.sqrt(bs)).astype(np.float32)
    g = None
    if fmt == "nvfp4":
        g = quant.nvfp4_tensor_scale(quant.apply_transform(T, X[_sample(n, 256, 5)]))
    sdt = torch.int16 if fmt == "int4" else torch.uint8
    xc = torch.empty((n, d_in // 2), dtype=torch.uint8, device=DEV)
    xs = torch.empty((n, d_in // bs), dtype=sdt, device=DEV)
    W.wush_transform_quant(fmt, to_dev(X), to_dev(T), xc, xs, g=g or 0.0)
    torch.cuda.synchronize()
    if fmt == "mxfp4":
        # the plane-ordered call (its own streamed kernel): the same codes, and scales equal to the
        # row-major ones re-laid by the library (both buffers zeroed first: rows past n stay zero)
        xc2 = torch.empty_like(xc)
        pa = torch.zeros(W.wush_mxfp4_planes_bytes(n, d_in), dtype=torch.uint8, device=DEV)
        pb = torch.zeros_like(pa)
        W.wush_transform_quant_mx_planes(to_dev(X), to_dev(T), xc2, pa)
        W.wush_mxfp4_scale_planes(xs, pb, d_in)
        torch.cuda.synchronize()
        assert torch.equal(xc2, xc)
        assert torch.equal(pa, pb)
        del xc2, pa, pb
    tok = _sample(n, 24, 6)
    rc, rs = quant.transform_quant(fmt, T, X[tok], g=g)
    assert np.array_equal(scales_np(xs, fmt)[tok], rs)
    assert np.array_equal(host(xc)[tok], rc)
