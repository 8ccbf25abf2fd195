"""GPU parity of every libwush device call against the oracle (small and ragged sizes).

Codes and scales must match bit-exactly; matmul outputs and the loss within
the relative tolerance 1e-3 (per element, against max(|ref|, rms(ref))).
The oracle builds its own transforms, codes and outputs from the seeded
inputs; nothing it consumes comes from the GPU.
"""

import numpy as np
import pytest
import torch

import aware_block_transforms_amd as W
from oracle import quant, transforms as tr, gemm as og, had256 as oh
from synth.gen import random_case, bf16_round
from gpu_util import DEV, to_dev, x_dev, host, scales_np, gemm_close

pytestmark = pytest.mark.gpu

SHAPES32 = [(1, 32), (200, 160), (130, 544), (64, 256)]
SHAPES16 = [(1, 16), (200, 208), (70, 48), (130, 256)]   # the last: four blocks per wave (NVFP4 merged stores)


def _oracle_tq(fmt, kind, X, Wt):
    bs = W.BLOCK[fmt]
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    Tx, Tw, _, _ = tr.build_transforms(kind, Wt, Sx, bs)
    ident = kind == "identity"
    g = None
    if fmt == "nvfp4":
        g = quant.nvfp4_tensor_scale(quant.apply_transform(Tx, X, identity=ident))
    c, s = quant.transform_quant(fmt, Tx, X, g=g, identity=ident)
    return Tx, Tw, g, c, s


def _gpu_tq(fmt, X, Tx, dtype, g, ident):
    n, d_in = X.shape
    bs = W.BLOCK[fmt]
    codes = torch.empty((n, d_in // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((n, d_in // bs), dtype=torch.int16 if fmt == "int4" else torch.uint8, device=DEV)
    W.wush_transform_quant(fmt, x_dev(X, dtype), None if ident else to_dev(Tx), codes, sc, g=g or 0.0)
    torch.cuda.synchronize()
    return host(codes), scales_np(sc, fmt)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["identity", "hadamard", "wus", "wush"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_transform_quant_bit_exact(fmt, kind, dtype):
    shapes = SHAPES16 if fmt == "nvfp4" else SHAPES32
    for si, (n, d_in) in enumerate(shapes):
        Wt, X = random_case(100 + si, n, d_in, 48, dtype=dtype)
        Tx, _, g, rc, rs = _oracle_tq(fmt, kind, X, Wt)
        gc, gs = _gpu_tq(fmt, X, Tx, dtype, g, kind == "identity")
        assert np.array_equal(gs, rs), (fmt, kind, dtype, n, d_in, np.argwhere(gs != rs)[:5])
        assert np.array_equal(gc, rc), (fmt, kind, dtype, n, d_in, np.argwhere(gc != rc)[:5])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [32, 16])
def test_transform_apply_bit_exact(bs, dtype):
    # the transformed values themselves, bit for bit (signed zeros included)
    fmt = "mxfp4" if bs == 32 else "nvfp4"
    for si, (n, d_in) in enumerate(SHAPES32 if bs == 32 else SHAPES16):
        Wt, X = random_case(300 + si, n, d_in, 40, dtype=dtype)
        for kind in ("hadamard", "wus", "wush"):
            Tx, _, _, _, _ = _oracle_tq(fmt, kind, X, Wt)
            Y = torch.empty((n, d_in), dtype=torch.float32, device=DEV)
            W.wush_transform_apply(x_dev(X, dtype), to_dev(Tx), Y)
            torch.cuda.synchronize()
            ref = quant.apply_transform(Tx, X)
            assert np.array_equal(host(Y).view(np.uint32), ref.view(np.uint32)), (bs, dtype, kind, n, d_in)


def _adversarial(rng, shape, lo, hi):
    # random signs and exponents spread over [lo, hi): wide dynamic range, so
    # that partial sums cancel and round differently in any other order
    e = rng.integers(lo, hi, size=shape)
    m = 1.0 + rng.random(shape)
    return (np.where(rng.random(shape) < 0.5, -1.0, 1.0) * np.ldexp(m, e)).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [32, 16])
def test_transform_apply_adversarial(bs, dtype):
    rng = np.random.default_rng([11, bs])
    n, d_in = 96, 8 * bs
    nblk = d_in // bs
    T = _adversarial(rng, (nblk, bs, bs), -30, 30)
    T[1] = _adversarial(rng, (bs, bs), -8, 8)
    T[1, :, bs // 2:] = -T[1, :, :bs // 2] * np.float32(1 + 2.0 ** -20)    # near-total cancellation
    X = _adversarial(rng, (n, d_in), -30, 30)
    X[:16] = _adversarial(rng, (16, d_in), -149, -120)                     # subnormal and tiny inputs
    X[16:32, : d_in // 2] = np.float32(0.0)
    X[16:32, d_in // 2:] = np.float32(-0.0)                               # signed zeros
    X[32:48] = _adversarial(rng, (16, d_in), -8, 8)
    X[32:48, bs // 2: bs] = X[32:48, : bs // 2]                            # pairs with the cancelling block
    if dtype == "bf16":
        X = bf16_round(X)
    Y = torch.empty((n, d_in), dtype=torch.float32, device=DEV)
    W.wush_transform_apply(x_dev(X, dtype), to_dev(T), Y)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        ref = quant.apply_transform(T, X)
    assert np.isfinite(ref).all()
    assert np.array_equal(host(Y).view(np.uint32), ref.view(np.uint32)), np.argwhere(host(Y) != ref)[:8]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_transform_quant_and_pack_shared_bit_exact(fmt, dtype):
    # shared-transform variant: block b uses its group's matrix; the oracle
    # expands the groups to per-block matrices and runs its own chain
    bs = W.BLOCK[fmt]
    for si, (n, d_in) in enumerate(SHAPES16 if bs == 16 else SHAPES32):
        Wt, X = random_case(500 + si, n, d_in, 40, dtype=dtype)
        nblk = d_in // bs
        ng = min(3, nblk)
        group = (np.arange(nblk) * 7 + si) % ng
        group[:ng] = np.arange(ng)                     # every group owns a block
        Sx = tr.activation_moments(X, bs).astype(np.float32)
        Tg, Twg, _, _ = tr.build_shared("wush", Wt, Sx, bs, group, ng)
        Tx, Tw = tr.expand_shared(Tg, group), tr.expand_shared(Twg, group)
        gdev = to_dev(group.astype(np.int32))
        g = None
        if fmt == "nvfp4":
            g = quant.nvfp4_tensor_scale(quant.apply_transform(Tx, X))
            g_dev = W.wush_nvfp4_global_scale_shared(x_dev(X, dtype), to_dev(Tg), gdev)
            assert np.float32(g_dev) == g
        rc, rs = quant.transform_quant(fmt, Tx, X, g=g)
        sdt = torch.int16 if fmt == "int4" else torch.uint8
        codes = torch.empty((n, d_in // 2), dtype=torch.uint8, device=DEV)
        sc = torch.empty((n, nblk), dtype=sdt, device=DEV)
        W.wush_transform_quant_shared(fmt, x_dev(X, dtype), to_dev(Tg), gdev, codes, sc, g=g or 0.0)
        torch.cuda.synchronize()
        assert np.array_equal(scales_np(sc, fmt), rs), (fmt, dtype, n, d_in)
        assert np.array_equal(host(codes), rc), (fmt, dtype, n, d_in)
        # weights
        gw = quant.nvfp4_tensor_scale(quant.apply_transform(Tw, Wt)) if fmt == "nvfp4" else None
        wc, ws_ = quant.transform_quant(fmt, Tw, Wt, g=gw)
        codes = torch.empty((Wt.shape[0], d_in // 2), dtype=torch.uint8, device=DEV)
        sc = torch.empty((Wt.shape[0], nblk), dtype=sdt, device=DEV)
        g_w = W.wush_pack_weights_shared(fmt, to_dev(Wt), to_dev(Twg), gdev, codes, sc)
        torch.cuda.synchronize()
        if fmt == "nvfp4":
            assert np.float32(g_w) == gw
        assert np.array_equal(scales_np(sc, fmt), ws_) and np.array_equal(host(codes), wc), (fmt, n, d_in)


@pytest.mark.parametrize("bs", [32, 16])
def test_build_transforms_on_device_equals_host_builder(bs):
    # same construction and fp64 operation order on both sides: identical matrices
    Wt, X = random_case(700 + bs, 300, 8 * bs, 96)
    Wt[:, bs:2 * bs] *= np.float32(1e-3)                    # a badly scaled block
    rng = np.random.default_rng(bs)
    Wt[:, 2 * bs:3 * bs] = np.outer(rng.standard_normal(Wt.shape[0]),
                                    rng.standard_normal(bs)).astype(np.float32)   # rank one: the damping ladder
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    nblk = Wt.shape[1] // bs
    for kind in ("identity", "hadamard", "wus", "wush"):
        hx = np.empty((nblk, bs, bs), np.float32)
        hw = np.empty_like(hx)
        W.wush_build_transforms(kind, bs, Wt, Sx, hx, hw)
        dx = torch.empty((nblk, bs, bs), dtype=torch.float32, device=DEV)
        dw = torch.empty_like(dx)
        W.wush_build_transforms_dev(kind, bs, to_dev(Wt), to_dev(Sx), dx, dw)
        ex, ew = host(dx), host(dw)
        ulp = lambda a, b: np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64)).max()
        assert np.array_equal(ex.view(np.uint32), hx.view(np.uint32)), (kind, ulp(ex, hx))
        assert np.array_equal(ew.view(np.uint32), hw.view(np.uint32)), (kind, ulp(ew, hw))
    Wz = Wt.copy()
    Wz[:, :bs] = 0.0                                        # all-zero block: no Cholesky factor at any rung
    dx = torch.empty((nblk, bs, bs), dtype=torch.float32, device=DEV)
    with pytest.raises(W.WushError) as e:
        W.wush_build_transforms_dev("wush", bs, to_dev(Wz), to_dev(Sx), dx, torch.empty_like(dx))
    assert e.value.status == W.WUSH_E_NUMERIC


@pytest.mark.parametrize("bs", [32, 16])
def test_build_transforms_on_device_matches_oracle(bs):
    # the device builder against the oracle's own construction (LAPACK Cholesky
    # and eigh in fp64): a few fp32 ulps of each block's largest entry and the
    # same proxy loss
    Wt, X = random_case(720 + bs, 400, 8 * bs, 112)
    Wt[:, bs:2 * bs] *= np.float32(1e-3)                    # a badly scaled block
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    nblk = Wt.shape[1] // bs
    A = tr.weight_moments(Wt, bs)
    for kind in ("identity", "hadamard", "wus", "wush"):
        dx = torch.empty((nblk, bs, bs), dtype=torch.float32, device=DEV)
        dw = torch.empty_like(dx)
        W.wush_build_transforms_dev(kind, bs, to_dev(Wt), to_dev(Sx), dx, dw)
        ex, ew = host(dx), host(dw)
        rx, rw, _, _ = tr.build_transforms(kind, Wt, Sx, bs)
        if kind in ("identity", "hadamard"):
            assert np.array_equal(ex, rx) and np.array_equal(ew, rw), kind
            continue
        for T, R in ((ex, rx), (ew, rw)):
            tol = 8 * 2.0 ** -24 * np.abs(R).max(axis=(1, 2), keepdims=True)
            assert np.all(np.abs(T - R) <= tol), (kind, np.abs(T - R).max())
        for b in range(nblk):
            j_d = tr.proxy_loss(ew[b].astype(np.float64), A[b], Sx[b].astype(np.float64))
            j_o = tr.proxy_loss(rw[b].astype(np.float64), A[b], Sx[b].astype(np.float64))
            assert np.isclose(j_d, j_o, rtol=1e-5), (kind, b)


def _planes_np(S):
    """Row-major E8M0 scales [rows][K/32] -> the matmul's plane order (layout of wush.h)."""
    rows, G = S.shape
    nb, tiles = G // 8, (rows + 255) // 256
    r = np.arange(rows)[:, None]
    gi = np.arange(G)[None, :]
    rr, b = r % 256, gi % 8
    pos = (8 * (rr // 128) + (rr // 16) % 8) ^ (8 * (b % 2))
    off = ((r // 256) * nb + gi // 8) * 2048 + b * 256 + (rr % 16) * 16 + pos
    P = np.zeros(tiles * nb * 2048, np.uint8)
    P[off.ravel()] = S.ravel()
    return P


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx_planes_path_matches_row_major_path(dtype):
    n, d_in, d_out = 300, 512, 320
    Wt, X = random_case(600, n, d_in, d_out, dtype=dtype)
    Tx, Tw, _, rc, rs = _oracle_tq("mxfp4", "wush", X, Wt)
    xd = x_dev(X, dtype)
    codes = torch.empty((n, d_in // 2), dtype=torch.uint8, device=DEV)
    pa = torch.zeros(W.wush_mxfp4_planes_bytes(n, d_in), dtype=torch.uint8, device=DEV)
    W.wush_transform_quant_mx_planes(xd, to_dev(Tx), codes, pa)
    wc = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=DEV)
    wsc = torch.empty((d_out, d_in // 32), dtype=torch.uint8, device=DEV)
    W.wush_pack_weights("mxfp4", to_dev(Wt), to_dev(Tw), wc, wsc)
    pb = torch.empty(W.wush_mxfp4_planes_bytes(d_out, d_in), dtype=torch.uint8, device=DEV)
    W.wush_mxfp4_scale_planes(wsc, pb, d_in)
    torch.cuda.synchronize()
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(pa), _planes_np(rs))                  # padding rows stay zero
    assert np.array_equal(host(pb), _planes_np(host(wsc)))
    # the matmul on plane-ordered scales equals the row-major call bit for bit
    xc = torch.empty_like(codes)
    xs = torch.empty((n, d_in // 32), dtype=torch.uint8, device=DEV)
    W.wush_transform_quant("mxfp4", xd, to_dev(Tx), xc, xs)
    Y0 = torch.empty((n, d_out), dtype=torch.float32, device=DEV)
    Y1 = torch.empty_like(Y0)
    W.wush_w4a4_gemm("mxfp4", xc, xs, wc, wsc, Y0)
    W.wush_w4a4_gemm_mx_planes(codes, pa, wc, pb, Y1)
    torch.cuda.synchronize()
    assert np.array_equal(host(Y0).view(np.uint32), host(Y1).view(np.uint32))


def _edge_inputs(d_in):
    rng = np.random.default_rng(77)
    X = rng.standard_normal((9, d_in)).astype(np.float32)
    X[0] = 0.0                                        # all-zero rows
    X[1] = -0.0
    X[2, :16] = np.float32(1e-40)                     # subnormal block
    X[3, 5] = np.float32(3e37)                        # huge value
    X[4] *= np.float32(2.0 ** -120)                   # tiny but normal
    X[5, ::2] = np.float32(6.0 * 2 ** -3)             # exact E2M1 grid points / ties
    X[5, 1::2] = np.float32(0.25 * 2 ** -3)
    X[6, 7] = np.nan                                  # NaN block
    X[7, 17] = np.inf                                 # Inf block
    X[8, :] = np.float32(1.0)
    return X


@pytest.mark.parametrize("kind", ["identity", "wush"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_transform_quant_edge_cases(fmt, kind):
    d_in = 64
    X = _edge_inputs(d_in)
    Wt, Xcal = random_case(5, 50, d_in, 40)
    bs = W.BLOCK[fmt]
    Sx = tr.activation_moments(Xcal, bs).astype(np.float32)
    Tx, _, _, _ = tr.build_transforms(kind, Wt, Sx, bs)
    ident = kind == "identity"
    g = np.float32(0.01) if fmt == "nvfp4" else None
    with np.errstate(all="ignore"):
        rc, rs = quant.transform_quant(fmt, Tx, X, g=g, identity=ident)
    gc, gs = _gpu_tq(fmt, X, Tx, "f32", g, ident)
    assert np.array_equal(gs, rs), np.argwhere(gs != rs)[:8]
    assert np.array_equal(gc, rc), np.argwhere(gc != rc)[:8]


# Hadamard-diagonal variant: 65 blocks (two 64-block lane groups, the second
# with one block) and 37 tokens (a ragged last wave) besides small shapes
SHAPES_HD = {32: [(1, 32), (200, 160), (37, 2080)], 16: [(1, 16), (70, 48), (37, 1040)]}


def _gpu_tq_hd(fmt, X, dx, dtype, g):
    n, d_in = X.shape
    bs = W.BLOCK[fmt]
    codes = torch.empty((n, d_in // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((n, d_in // bs), dtype=torch.int16 if fmt == "int4" else torch.uint8, device=DEV)
    W.wush_transform_quant_hd(fmt, x_dev(X, dtype), to_dev(dx), codes, sc, g=g or 0.0)
    torch.cuda.synchronize()
    return host(codes), scales_np(sc, fmt)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_transform_quant_hd_bit_exact(fmt, dtype):
    bs = W.BLOCK[fmt]
    for si, (n, d_in) in enumerate(SHAPES_HD[bs]):
        Wt, X = random_case(300 + si, n, d_in, 48, dtype=dtype)
        Sx = tr.activation_moments(X, bs).astype(np.float32)
        dx, _, _, _ = tr.build_hd(Wt, Sx, bs)
        g = quant.nvfp4_tensor_scale(quant.apply_hd(dx, X, bs)) if fmt == "nvfp4" else None
        rc, rs = quant.transform_quant_hd(fmt, dx, X, g=g)
        gc, gs = _gpu_tq_hd(fmt, X, dx, dtype, g)
        assert np.array_equal(gs, rs), (fmt, dtype, n, d_in, np.argwhere(gs != rs)[:5])
        assert np.array_equal(gc, rc), (fmt, dtype, n, d_in, np.argwhere(gc != rc)[:5])


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_transform_quant_hd_edge_cases(fmt):
    d_in = 64
    X = _edge_inputs(d_in)
    Wt, Xcal = random_case(6, 50, d_in, 40)
    bs = W.BLOCK[fmt]
    dx, _, _, _ = tr.build_hd(Wt, tr.activation_moments(Xcal, bs).astype(np.float32), bs)
    g = np.float32(0.01) if fmt == "nvfp4" else None
    with np.errstate(all="ignore"):
        rc, rs = quant.transform_quant_hd(fmt, dx, X, g=g)
    gc, gs = _gpu_tq_hd(fmt, X, dx, "f32", g)
    assert np.array_equal(gs, rs), np.argwhere(gs != rs)[:8]
    assert np.array_equal(gc, rc), np.argwhere(gc != rc)[:8]


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_pack_weights_hd_and_tensor_scale_bit_exact(fmt):
    bs = W.BLOCK[fmt]
    Wt, X = random_case(9, 300, 2080 if bs == 32 else 1040, 77)
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    dx, dw, _, _ = tr.build_hd(Wt, Sx, bs)
    g = quant.nvfp4_tensor_scale(quant.apply_hd(dw, Wt, bs)) if fmt == "nvfp4" else None
    rc, rs = quant.transform_quant_hd(fmt, dw, Wt, g=g)
    d_out, d_in = Wt.shape
    codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((d_out, d_in // bs), dtype=torch.int16 if fmt == "int4" else torch.uint8, device=DEV)
    gg = W.wush_pack_weights_hd(fmt, to_dev(Wt), to_dev(dw), codes, sc)
    torch.cuda.synchronize()
    if fmt == "nvfp4":
        assert np.float32(gg).view(np.uint32) == np.float32(g).view(np.uint32)
        # and the activation-side tensor scale, bf16 input
        Xb = X[:64]
        ref = quant.nvfp4_tensor_scale(quant.apply_hd(dx, Xb, bs))
        ga = W.wush_nvfp4_global_scale_hd(x_dev(Xb, "f32"), to_dev(dx))
        assert np.float32(ga).view(np.uint32) == np.float32(ref).view(np.uint32)
    assert np.array_equal(scales_np(sc, fmt), rs)
    assert np.array_equal(host(codes), rc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [16, 32])
def test_block_moments_on_device(bs, dtype):
    # 1, 300 (two chunks, the second short) and 5000 tokens (20 chunks)
    for n in (1, 300, 5000):
        _, X = random_case(60 + n, n, 4 * bs + 64, 8, dtype=dtype)
        d_in = X.shape[1]
        Sx = torch.full((d_in // bs, bs, bs), np.nan, dtype=torch.float32, device=DEV)
        ws = torch.empty(W.wush_block_moments_dev_ws_bytes(bs, n, d_in), dtype=torch.uint8, device=DEV)
        for w in (None, ws):
            W.wush_block_moments_dev(bs, x_dev(X, dtype), Sx, ws=w)
            torch.cuda.synchronize()
            got = host(Sx)
            ref = tr.activation_moments(X, bs)
            assert np.array_equal(got, got.transpose(0, 2, 1))
            assert np.allclose(got, ref, rtol=2e-7, atol=1e-7 * np.abs(ref).max()), (n, np.abs(got - ref).max())
            # and the host library's fp64 moments up to summation order: within one fp32 ulp
            hx = np.empty_like(got)
            W.wush_block_moments(bs, X, hx)
            assert np.all(np.abs(got - hx) <= np.spacing(np.abs(hx)))


def test_transform_quant_empty_batch():
    codes = torch.empty((0, 16), dtype=torch.uint8, device=DEV)
    sc = torch.empty((0, 1), dtype=torch.uint8, device=DEV)
    X = torch.empty((0, 32), dtype=torch.float32, device=DEV)
    W.wush_transform_quant("mxfp4", X, None, codes, sc)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nvfp4_global_scale(dtype):
    Wt, X = random_case(7, 150, 96, 32, dtype=dtype)
    Sx = tr.activation_moments(X, 16).astype(np.float32)
    Tx, _, _, _ = tr.build_transforms("wush", Wt, Sx, 16)
    ref = quant.nvfp4_tensor_scale(quant.apply_transform(Tx, X))
    g = W.wush_nvfp4_global_scale(x_dev(X, dtype), to_dev(Tx))
    assert np.float32(g).view(np.uint32) == np.float32(ref).view(np.uint32)


@pytest.mark.parametrize("kind", ["identity", "wush"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_pack_weights_bit_exact(fmt, kind):
    Wt, X = random_case(8, 300, 160 if fmt != "nvfp4" else 176, 77)
    bs = W.BLOCK[fmt]
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    _, Tw, _, _ = tr.build_transforms(kind, Wt, Sx, bs)
    ident = kind == "identity"
    g = None
    if fmt == "nvfp4":
        g = quant.nvfp4_tensor_scale(quant.apply_transform(Tw, Wt, identity=ident))
    rc, rs = quant.transform_quant(fmt, Tw, Wt, g=g, identity=ident)
    d_out, d_in = Wt.shape
    codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((d_out, d_in // bs), dtype=torch.int16 if fmt == "int4" else torch.uint8, device=DEV)
    gg = W.wush_pack_weights(fmt, to_dev(Wt), None if ident else to_dev(Tw), codes, sc)
    torch.cuda.synchronize()
    assert np.array_equal(scales_np(sc, fmt), rs)
    assert np.array_equal(host(codes), rc)
    if fmt == "nvfp4":
        assert np.float32(gg) == g


# the LDS-staged kernel handles every K % 128 == 0; K / 128 steps cover the
# pipeline's cases (1, 2, 3 steps; whole groups of 4; groups plus 1-3 extra)
GEMM_SHAPES = [(16, 16, 128), (100, 70, 384), (257, 129, 640), (128, 256, 256), (64, 512, 1024),
               (300, 520, 512), (17, 300, 768), (1000, 260, 2048), (512, 1024, 4096), (260, 513, 1152),
               (33, 800, 1408)]


def _rand_operands(fmt, M, N, K, seed):
    rng = np.random.default_rng([seed, M, N, K])
    A = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1)))).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A[:, rng.choice(K, 3, replace=False)] *= 30
    ga = gb = None
    if fmt == "nvfp4":
        ga, gb = quant.nvfp4_tensor_scale(A), quant.nvfp4_tensor_scale(B)
    ca, sa = quant.transform_quant(fmt, None, A, g=ga, identity=True)
    cb, sb = quant.transform_quant(fmt, None, B, g=gb, identity=True)
    return ca, sa, cb, sb, ga, gb


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_w4a4_gemm(fmt, shape):
    M, N, K = shape
    ca, sa, cb, sb, ga, gb = _rand_operands(fmt, M, N, K, 1)
    ref = og.w4a4_gemm(fmt, ca, sa, cb, sb, ga, gb)
    # both scratch paths: library-taken (ws None) and a caller workspace filled with junk
    need = W.wush_w4a4_gemm_ws_bytes(fmt, M, N, K)
    ws = torch.full((need + 64,), 0xA5, dtype=torch.uint8, device=DEV) if need else None
    for w in (None, ws):
        Y = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
        W.wush_w4a4_gemm(fmt, to_dev(ca), to_dev(sa), to_dev(cb), to_dev(sb), Y,
                         a_g=ga or 1.0, b_g=gb or 1.0, ws=w)
        torch.cuda.synchronize()
        ok, worst = gemm_close(host(Y), ref)
        assert ok, (fmt, shape, w is None, worst)


@pytest.mark.parametrize("shape", [(4600, 4090, 1024), (250, 66001, 1024)])
def test_w4a4_gemm_more_tiles_than_workgroups(shape):
    # more 256 x 256 output tiles than compute units: the MXFP4 kernel's
    # workgroups each walk several tiles, with the loads of a tile's last
    # blocks fetching the next tile's first ones; ragged M and N (N % 4 != 0)
    M, N, K = shape
    ca, sa, cb, sb, _, _ = _rand_operands("mxfp4", M, N, K, 3)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    ref = og.w4a4_gemm_rows("mxfp4", rows, ca, sa, cb, sb)
    Y = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
    W.wush_w4a4_gemm("mxfp4", to_dev(ca), to_dev(sa), to_dev(cb), to_dev(sb), Y)
    torch.cuda.synchronize()
    Yh = host(Y)
    assert not np.isnan(Yh).any()
    ok, worst = gemm_close(Yh[rows], ref)
    assert ok, (shape, worst)


def test_w4a4_gemm_workspace_checks():
    M, N, K = 300, 260, 512
    ca, sa, cb, sb, _, _ = _rand_operands("mxfp4", M, N, K, 2)
    need = W.wush_w4a4_gemm_ws_bytes("mxfp4", M, N, K)
    assert need == (2 + 2) * 2 * 2048            # (row tiles of A + of B) x K blocks x 2 KB
    assert W.wush_w4a4_gemm_ws_bytes("mxfp4", M, N, 128) == 0   # K = 128: direct kernel, no scratch
    # NVFP4: 16 fp16 scale planes of 256 entries per (row tile, K block)
    assert W.wush_w4a4_gemm_ws_bytes("nvfp4", M, N, K) == (2 + 2) * 2 * 8192
    # INT4: fp32 scales, 8 per row and K block (256-row A tiles, 128-row B tiles)
    assert W.wush_w4a4_gemm_ws_bytes("int4", M, N, K) == 2 * (2 * 8192 + 3 * 4096)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(W.WushError):
        W.wush_w4a4_gemm("mxfp4", to_dev(ca), to_dev(sa), to_dev(cb), to_dev(sb), Y, ws=small)
    ca, sa, cb, sb, ga, gb = _rand_operands("nvfp4", M, N, K, 2)
    small = torch.empty(W.wush_w4a4_gemm_ws_bytes("nvfp4", M, N, K) - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(W.WushError):
        W.wush_w4a4_gemm("nvfp4", to_dev(ca), to_dev(sa), to_dev(cb), to_dev(sb), Y, a_g=ga, b_g=gb, ws=small)
    ca, sa, cb, sb, _, _ = _rand_operands("int4", M, N, K, 2)
    small = torch.empty(W.wush_w4a4_gemm_ws_bytes("int4", M, N, K) - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(W.WushError):
        W.wush_w4a4_gemm("int4", to_dev(ca), to_dev(sa), to_dev(cb), to_dev(sb), Y, ws=small)


def test_layer_loss():
    rng = np.random.default_rng(3)
    for M, N in [(1, 1), (3, 5), (128, 256), (333, 77)]:
        Yh = rng.standard_normal((M, N)).astype(np.float32)
        Yr = (Yh + rng.standard_normal((M, N)) * 0.1).astype(np.float32)
        ref = og.layer_loss(Yh, Yr)
        ws = torch.empty(W.wush_loss_ws_bytes(M, N) // 8, dtype=torch.float64, device=DEV)
        out = torch.empty(1, dtype=torch.float64, device=DEV)
        W.wush_layer_loss(to_dev(Yh), to_dev(Yr), out, ws)
        torch.cuda.synchronize()
        assert abs(out.item() - ref) <= 1e-3 * ref, (M, N, out.item(), ref)
        # deterministic: same bits on a second call
        out2 = torch.empty(1, dtype=torch.float64, device=DEV)
        W.wush_layer_loss(to_dev(Yh), to_dev(Yr), out2, ws)
        torch.cuda.synchronize()
        assert out.item() == out2.item()


def test_had256_pack_bit_exact_and_rotate():
    # 37 rows: two full 16-row blocks and one with 11 padding rows
    Wt, _ = random_case(30, 1, 768, 37)
    packed = torch.full((W.wush_had256_packed_bytes(37, 768),), 0xA5, dtype=torch.uint8, device=DEV)
    W.wush_had256_pack_weights(to_dev(Wt), packed)
    ref = oh.pack_weights(Wt)
    torch.cuda.synchronize()
    assert packed.numel() == ref.size
    assert np.array_equal(host(packed).reshape(ref.shape), ref)
    # rotation equals the oracle's butterflies bit for bit; two rotations are exact on integers
    out = torch.empty((37, 768), dtype=torch.float32, device=DEV)
    W.wush_had256_rotate(to_dev(Wt), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), oh.fwht256(Wt.reshape(37, 3, 256)).reshape(37, 768).view(np.uint32))
    ints = np.random.default_rng(4).integers(-2 ** 15, 2 ** 15 + 1, (5, 512)).astype(np.float32)
    a = to_dev(ints)
    W.wush_had256_rotate(a, a)
    W.wush_had256_rotate(a, a)
    torch.cuda.synchronize()
    assert np.array_equal(host(a), ints)


# d_in 1280 = 5 chunks (fewer than the 16 waves of a workgroup), 5120 = 20
# chunks (a second pass for four waves); d_out 200 = 12.5 row blocks: a
# padded last block and a last workgroup with one of its four blocks
@pytest.mark.parametrize("batch,d_in", [(1, 1280), (3, 1280), (4, 1280), (5, 1280), (16, 1280), (1, 5120),
                                        (16, 5120)])
def test_had256_gemv(batch, d_in):
    Wt, _ = random_case(31, 1, d_in, 200)
    rp = oh.pack_weights(Wt)
    x = np.random.default_rng(batch).standard_normal((batch, d_in)).astype(np.float32)
    from synth.gen import bf16_round, bf16_bits
    xb = bf16_round(x)
    ref = oh.gemv(xb, rp, 200)
    ws = torch.full((W.wush_had256_gemv_ws_bytes(batch, d_in),), 0x5A, dtype=torch.uint8, device=DEV)
    for w in (None, ws):
        y = torch.full((batch, 200), np.nan, dtype=torch.float32, device=DEV)
        W.wush_had256_gemv(to_dev(bf16_bits(xb).view(np.int16)), to_dev(rp.reshape(-1)), y, ws=w)
        torch.cuda.synchronize()
        ok, worst = gemm_close(host(y), ref)
        assert ok, (w is None, worst)


@pytest.mark.parametrize("fmt,kind", [("mxfp4", "wush"), ("nvfp4", "wus"), ("int4", "hadamard"), ("mxfp4", "identity")])
def test_w4a4_layer_helper_matches_oracle(fmt, kind):
    # aware_block_transforms_amd.layer.W4A4Layer: host-built transforms, packed
    # weights, then quantize + matmul through the library calls
    from aware_block_transforms_amd.layer import W4A4Layer
    bs = W.BLOCK[fmt]
    Wt, X = random_case(810, 150, 256, 200)
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    Tx, Tw, _, _ = tr.build_transforms(kind, Wt, Sx, bs)     # the oracle's pair, fed to both sides
    L = W4A4Layer(fmt, kind, Wt, Tx=Tx, Tw=Tw)
    Xd = to_dev(X)
    ident = kind == "identity"
    gx = None
    if fmt == "nvfp4":
        assert np.float32(L.calibrate(Xd)) == quant.nvfp4_tensor_scale(quant.apply_transform(Tx, X, identity=ident))
        gx = np.float32(L.x_g)
    gw = quant.nvfp4_tensor_scale(quant.apply_transform(Tw, Wt, identity=ident)) if fmt == "nvfp4" else None
    wc, ws_ = quant.transform_quant(fmt, Tw, Wt, g=gw, identity=ident)
    assert np.array_equal(host(L.w_codes), wc) and np.array_equal(scales_np(L.w_scales, fmt), ws_)
    Y = L.forward(Xd)
    torch.cuda.synchronize()
    xc, xs = quant.transform_quant(fmt, Tx, X, g=gx, identity=ident)
    ok, worst = gemm_close(host(Y), og.w4a4_gemm(fmt, xc, xs, wc, ws_, gx, gw))
    assert ok, (fmt, kind, worst)
