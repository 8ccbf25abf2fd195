"""CPU tests of the C ABI: the library loads, exports every declared symbol,
rejects bad arguments before touching the GPU, and its host-side builder and
moment accumulation agree with the oracle."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wush.h")

W = pytest.importorskip("aware_block_transforms_amd._lib")
from oracle import transforms as tr  # noqa: E402
from synth.gen import random_case, CONFIGS, make_weights, make_activations  # noqa: E402


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wush_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 14
    for name in names:
        assert hasattr(W.lib, name), name
    # and the binding wraps each of them
    assert set(names) <= set(W.EXPORTED), set(names) - set(W.EXPORTED)


def test_status_strings_and_version():
    assert W.lib.wush_status_string(0) == b"ok"
    assert W.lib.wush_status_string(3) == b"numerical failure"
    assert W.wush_version().startswith("wush")
    assert W.lib.wush_format_block(0) == 32 and W.lib.wush_format_block(1) == 16
    assert W.lib.wush_format_block(2) == 32 and W.lib.wush_format_block(7) == 0


def test_device_calls_reject_bad_arguments_before_launch():
    L = W.lib
    # null pointers / bad shapes / bad enums: validated on the host, no HIP call made
    assert L.wush_transform_quant(0, 0, 4, 64, None, None, 0.0, None, None, None) == W.WUSH_E_ARG
    assert L.wush_transform_quant(0, 0, 4, 63, None, None, 0.0, None, None, None) == W.WUSH_E_SHAPE
    assert L.wush_transform_quant(9, 0, 4, 64, None, None, 0.0, None, None, None) == W.WUSH_E_ARG
    assert b"format" in L.wush_last_error()
    assert L.wush_transform_apply(0, 24, 4, 64, None, None, None, None) == W.WUSH_E_ARG
    assert L.wush_transform_apply(0, 32, 4, 48, None, None, None, None) == W.WUSH_E_SHAPE
    assert L.wush_transform_apply(0, 32, 4, 64, None, None, None, None) == W.WUSH_E_ARG
    assert L.wush_transform_apply(0, 32, 0, 64, None, None, None, None) == W.WUSH_OK
    assert L.wush_w4a4_gemm(0, 4, 4, 100, None, None, 1.0, None, None, 1.0, None, None, 0, None) == W.WUSH_E_SHAPE
    assert L.wush_w4a4_gemm(0, 4, 4, 128, None, None, 1.0, None, None, 1.0, None, None, 0, None) == W.WUSH_E_ARG
    assert L.wush_w4a4_gemm(0, 0, 4, 128, None, None, 1.0, None, None, 1.0, None, None, 0, None) == W.WUSH_E_SHAPE
    assert L.wush_layer_loss(0, 4, None, None, None, None, None) == W.WUSH_E_ARG
    assert L.wush_had256_gemv(17, 4, 256, None, None, None, None, 0, None) == W.WUSH_E_SHAPE
    assert L.wush_had256_gemv(1, 4, (1 << 24) + 256, None, None, None, None, 0, None) == W.WUSH_E_SHAPE
    assert L.wush_had256_gemv(1, 4, 256, None, None, None, None, 0, None) == W.WUSH_E_ARG
    # workspace sizes (host-side arithmetic only)
    assert L.wush_had256_gemv_ws_bytes(5, 4096) == 2 * 5 * 4096 + 5 * 16 * 16
    assert L.wush_had256_gemv_ws_bytes(4, 4096) == 0    # batches up to 4 rotate inside the GEMV
    assert L.wush_had256_packed_bytes(37, 768) == 3 * 3 * 1568       # rows padded to 16-row blocks
    assert L.wush_had256_packed_bytes(14336, 4096) == 896 * 16 * 1568
    assert L.wush_had256_packed_bytes(4, 100) == 0
    assert L.wush_had256_gemv_ws_bytes(0, 4096) == 0
    assert L.wush_had256_gemv_ws_bytes(1, 4096) == 0
    assert L.wush_w4a4_gemm_ws_bytes(0, 4096, 12288, 4096) == (16 + 48) * 16 * 2048
    assert L.wush_w4a4_gemm_ws_bytes(0, 4096, 12288, 128) == 0
    assert L.wush_w4a4_gemm_ws_bytes(1, 4096, 12288, 4096) == (16 + 48) * 16 * 8192
    assert L.wush_w4a4_gemm_ws_bytes(1, 4096, 12288, 128) == (16 + 48) * 1 * 8192
    assert L.wush_w4a4_gemm_ws_bytes(2, 4096, 12288, 4096) == 16 * (16 * 8192 + 96 * 4096)
    assert L.wush_had256_pack_weights(4, 100, None, None, None) == W.WUSH_E_SHAPE
    assert L.wush_had256_pack_weights(4, 256, None, None, None) == W.WUSH_E_ARG
    assert L.wush_had256_rotate(4, 256, None, None, None) == W.WUSH_E_ARG
    assert L.wush_loss_ws_bytes(10, 10) >= 8
    # misaligned pointer
    buf = np.zeros(64, np.uint8)
    assert L.wush_transform_quant(0, 0, 1, 32, buf.ctypes.data + 1, None, 0.0, buf.ctypes.data, buf.ctypes.data,
                                  None) == W.WUSH_E_ARG
    # NVFP4 needs a positive finite tensor scale
    assert L.wush_transform_quant(1, 0, 1, 32, buf.ctypes.data, None, 0.0, buf.ctypes.data, buf.ctypes.data,
                                  None) == W.WUSH_E_ARG


def test_builder_rejects_bad_input():
    T = np.zeros((2, 32, 32), np.float32)
    with pytest.raises(W.WushError) as e:
        W.wush_build_transforms("wush", 32, None, None, T, T.copy())
    assert e.value.status == W.WUSH_E_ARG
    Wt = np.zeros((4, 64), np.float32)
    with pytest.raises(W.WushError) as e:
        W.wush_build_transforms("wush", 24, Wt, np.zeros((2, 32, 32), np.float32), T, T.copy())
    assert e.value.status == W.WUSH_E_SHAPE


def test_builder_damps_rank_deficient_blocks_like_the_oracle():
    rng = np.random.default_rng(3)
    Wt = rng.standard_normal((8, 64)).astype(np.float32)       # 8 rows: rank-deficient 32x32 moments
    X = rng.standard_normal((100, 64)).astype(np.float32)
    Sx = tr.activation_moments(X, 32).astype(np.float32)
    Tx = np.empty((2, 32, 32), np.float32)
    Tw = np.empty_like(Tx)
    W.wush_build_transforms("wush", 32, Wt, Sx, Tx, Tw)
    _, _, tx64, tw64 = tr.build_transforms("wush", Wt, Sx, 32)
    for b in range(2):
        assert np.allclose(Tw[b].astype(np.float64).T @ Tx[b].astype(np.float64), np.eye(32), atol=1e-3)
    assert np.allclose(Tx, tx64, rtol=1e-3, atol=1e-3 * np.abs(tx64).max())


def test_builder_zero_weights_is_numeric_error():
    Wt = np.zeros((16, 32), np.float32)
    Sx = np.eye(32, dtype=np.float32)[None]
    T = np.empty((1, 32, 32), np.float32)
    with pytest.raises(W.WushError) as e:
        W.wush_build_transforms("wush", 32, Wt, Sx, T, T.copy())
    assert e.value.status == W.WUSH_E_NUMERIC


def test_moments_match_oracle():
    _, X = random_case(21, 300, 128, 8)
    for bs in (16, 32):
        Sx = np.empty((128 // bs, bs, bs), np.float32)
        W.wush_block_moments(bs, X, Sx)
        ref = tr.activation_moments(X, bs)
        assert np.allclose(Sx, ref, rtol=2e-7, atol=1e-7 * np.abs(ref).max())
        assert np.array_equal(Sx, Sx.transpose(0, 2, 1))


def _t_tolerance(T, ref):
    # the two builders round the same fp64 matrix to fp32 from slightly different
    # fp64 values (Jacobi vs LAPACK eigh, different summation orders); allow a
    # few fp32 ulps of the block's largest entry
    return 8 * 2.0 ** -24 * np.abs(ref).max(axis=(1, 2), keepdims=True)


@pytest.mark.parametrize("kind", ["identity", "hadamard", "wus", "wush"])
@pytest.mark.parametrize("bs", [16, 32])
def test_builder_matches_oracle(kind, bs):
    Wt, X = random_case(22 + bs, 400, 256, 96)
    Sx = tr.activation_moments(X, bs).astype(np.float32)
    nblk = 256 // bs
    Tx = np.empty((nblk, bs, bs), np.float32)
    Tw = np.empty_like(Tx)
    W.wush_build_transforms(kind, bs, Wt, Sx, Tx, Tw)
    rx, rw, _, _ = tr.build_transforms(kind, Wt, Sx, bs)
    if kind in ("identity", "hadamard"):
        assert np.array_equal(Tx, rx) and np.array_equal(Tw, rw)
        return
    assert np.all(np.abs(Tx - rx) <= _t_tolerance(Tx, rx)), np.abs(Tx - rx).max()
    assert np.all(np.abs(Tw - rw) <= _t_tolerance(Tw, rw)), np.abs(Tw - rw).max()
    # proxy loss equal to the closed form to high accuracy
    A = tr.weight_moments(Wt, bs)
    for b in range(nblk):
        j_c = tr.proxy_loss(Tw[b].astype(np.float64), A[b], Sx[b].astype(np.float64))
        j_o = tr.proxy_loss(rw[b].astype(np.float64), A[b], Sx[b].astype(np.float64))
        assert np.isclose(j_c, j_o, rtol=1e-5)


def test_builder_on_tiny_workload():
    w = CONFIGS["tiny"]
    Wt = make_weights(w)
    X = make_activations(w)
    Sx = np.empty((8, 32, 32), np.float32)
    W.wush_block_moments(32, X, Sx)
    Tx = np.empty((8, 32, 32), np.float32)
    Tw = np.empty_like(Tx)
    W.wush_build_transforms("wush", 32, Wt, Sx, Tx, Tw)
    rx, rw, _, _ = tr.build_transforms("wush", Wt, tr.activation_moments(X, 32).astype(np.float32), 32)
    assert np.all(np.abs(Tx - rx) <= _t_tolerance(Tx, rx) + 4 * 2.0 ** -24 * np.abs(rx).max())


def test_dma_kernels_leave_m0_to_their_dma():
    """The NVFP4 and INT4 kernels set M0 in inline asm just before each
    buffer_load ... lds (the compiler cannot see that write); no other
    instruction of theirs may read or write M0."""
    import re
    import subprocess
    from aware_block_transforms_amd import build as B
    for src in ("gemm_nvfp4.hip", "gemm_int4.hip"):
        r = subprocess.run([B.HIPCC, *B.HIP_FLAGS, "--cuda-device-only", "-S", "-o", "-",
                            os.path.join(B.CSRC, src)], capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = [l.strip() for l in r.stdout.splitlines()]
        code = [l for l in lines if l and not l.startswith((";", ".", "//")) and "ASM" not in l]
        n_dma = 0
        for i, l in enumerate(code):
            if not re.search(r"\bm0\b", l):
                continue
            assert re.match(r"s_mov_b32 m0, s\d+$", l), (src, l)
            assert re.match(r"buffer_load_dwordx4 .* offen lds$", code[i + 1]), (src, l, code[i + 1])
            n_dma += 1
        assert n_dma > 0, src


def test_build_hd_matches_oracle_and_rejects_bad_input():
    W_, X = random_case(41, 300, 128, 64)
    for bs in (16, 32):
        Sx = tr.activation_moments(X, bs).astype(np.float32)
        Sx[0, 3, 3] = 0.0                         # a dead activation channel is floored, not infinite
        dx = np.empty(128, np.float32)
        dw = np.empty(128, np.float32)
        W.wush_build_hd(bs, W_, Sx, dx, dw)
        rx, rw, rx64, rw64 = tr.build_hd(W_, Sx, bs)
        # both round the same fp64 values (summed in different orders) to fp32
        assert np.allclose(dx, rx64, rtol=4 * 2.0 ** -24, atol=0) and np.allclose(dw, rw64, rtol=4 * 2.0 ** -24, atol=0)
        assert np.all(np.isfinite(dx)) and np.all(dx > 0)
    Wz = W_.copy()
    Wz[:, :32] = 0.0                              # a block with all-zero weights
    with pytest.raises(W.WushError) as e:
        W.wush_build_hd(32, Wz, Sx, dx, dw)
    assert e.value.status == W.WUSH_E_NUMERIC
    L = W.lib
    assert L.wush_build_hd(24, 128, 64, None, None, None, None) == W.WUSH_E_ARG
    buf = np.zeros(4096, np.float32)
    p = buf.ctypes.data
    assert L.wush_build_hd(24, 96, 4, p, p, p, p) == W.WUSH_E_SHAPE
    assert L.wush_build_hd(32, 100, 4, p, p, p, p) == W.WUSH_E_SHAPE
    assert L.wush_transform_quant_hd(0, 0, 4, 100, None, None, 0.0, None, None, None) == W.WUSH_E_SHAPE
    assert L.wush_transform_quant_hd(0, 0, 4, 128, None, None, 0.0, None, None, None) == W.WUSH_E_ARG
    assert L.wush_pack_weights_hd(0, 4, 128, None, None, None, None, None, None) == W.WUSH_E_ARG
    assert L.wush_nvfp4_global_scale_hd(0, 4, 128, None, None, None, None) == W.WUSH_E_ARG


def test_build_shared_matches_oracle_and_rejects_bad_groups():
    W_, X = random_case(46, 200, 256, 48)
    for bs, group, ng in ((32, np.array([0, 1, 0, 2, 2, 1, 0, 1]), 3), (16, np.arange(16) % 5, 5),
                          (32, np.zeros(8, dtype=np.int32), 1)):
        Sx = tr.activation_moments(X, bs).astype(np.float32)
        for kind in ("wus", "wush", "hadamard"):
            Tx, Tw = W.wush_build_shared(kind, W_, Sx, bs, group, ng)
            _, _, rx, rw = tr.build_shared(kind, W_, Sx, bs, group, ng)
            # fp64 on both sides, summed in different orders, rounded to fp32:
            # within 8 fp32 ulps of each group matrix's largest entry
            for T, R in ((Tx, rx), (Tw, rw)):
                tol = 8 * 2.0 ** -24 * np.abs(R).reshape(ng, -1).max(axis=1)[:, None, None]
                assert np.all(np.abs(T - R) <= tol), (bs, kind)
    L = W.lib
    g = np.array([0, 1, 0, 3], dtype=np.int32)        # group 2 owns no block, 3 is out of range
    buf = np.zeros(8192, np.float32)
    p = buf.ctypes.data
    assert L.wush_build_shared(3, 32, 128, 4, p, p, 3, g.ctypes.data, p, p) == W.WUSH_E_ARG
    g = np.array([0, 1, 0, 0], dtype=np.int32)        # group 2 empty
    assert L.wush_build_shared(3, 32, 128, 4, p, p, 3, g.ctypes.data, p, p) == W.WUSH_E_ARG
    assert b"owns no block" in L.wush_last_error()
    assert L.wush_build_shared(3, 32, 128, 4, p, p, 5, g.ctypes.data, p, p) == W.WUSH_E_ARG
    assert L.wush_build_shared(3, 24, 128, 4, p, p, 1, g.ctypes.data, p, p) == W.WUSH_E_SHAPE
    assert L.wush_transform_quant_shared(0, 0, 4, 128, None, None, 1, None, 0.0, None, None, None) == W.WUSH_E_ARG
    assert L.wush_transform_quant_shared(0, 0, 4, 100, None, None, 1, None, 0.0, None, None, None) == W.WUSH_E_SHAPE
    assert L.wush_pack_weights_shared(0, 4, 128, None, None, 1, None, None, None, None, None) == W.WUSH_E_ARG
    assert L.wush_nvfp4_global_scale_shared(0, 4, 128, None, None, 1, None, None, None) == W.WUSH_E_ARG


def test_build_transforms_dev_workspace_and_argument_checks():
    L = W.lib
    assert L.wush_build_transforms_dev_ws_bytes(32, 4096) == 128 * 32 * 32 * 8 + 512
    assert L.wush_build_transforms_dev_ws_bytes(16, 48) == 3 * 16 * 16 * 8 + 256
    assert L.wush_build_transforms_dev_ws_bytes(24, 48) == 0 and L.wush_build_transforms_dev_ws_bytes(32, 48) == 0
    buf = np.zeros(1 << 16, np.uint8)
    p = (buf.ctypes.data + 15) // 16 * 16
    assert L.wush_build_transforms_dev(9, 32, 64, 4, p, p, p, p, p, 1 << 15, None) == W.WUSH_E_ARG
    assert L.wush_build_transforms_dev(3, 24, 48, 4, p, p, p, p, p, 1 << 15, None) == W.WUSH_E_SHAPE
    assert L.wush_build_transforms_dev(3, 32, 64, 4, p, p, None, p, p, 1 << 15, None) == W.WUSH_E_ARG
    assert L.wush_build_transforms_dev(3, 32, 64, 4, None, p, p, p, p, 1 << 15, None) == W.WUSH_E_ARG
    assert L.wush_build_transforms_dev(3, 32, 64, 4, p, p, p, p, p, 100, None) == W.WUSH_E_ARG   # short workspace
    assert L.wush_build_transforms_dev(3, 32, 64, 4, p, p, p, p, None, 1 << 15, None) == W.WUSH_E_ARG


def test_mx_planes_sizes_and_argument_checks():
    L = W.lib
    assert L.wush_mxfp4_planes_bytes(300, 512) == 2 * 2 * 2048
    assert L.wush_mxfp4_planes_bytes(4096, 4096) == 16 * 16 * 2048
    assert L.wush_mxfp4_planes_bytes(10, 384) == 0 and L.wush_mxfp4_planes_bytes(0, 512) == 0
    assert L.wush_mxfp4_scale_planes(10, 384, None, None, None) == W.WUSH_E_SHAPE
    assert L.wush_mxfp4_scale_planes(10, 512, None, None, None) == W.WUSH_E_ARG
    assert L.wush_transform_quant_mx_planes(1, 4, 384, None, None, None, None, None) == W.WUSH_E_ARG
    buf = np.zeros(8192, np.uint8)
    p = (buf.ctypes.data + 15) // 16 * 16
    assert L.wush_transform_quant_mx_planes(1, 4, 384, p, p, p, p, None) == W.WUSH_E_SHAPE
    assert L.wush_transform_quant_mx_planes(1, 4, 512, p, None, p, p, None) == W.WUSH_E_ARG
    assert L.wush_w4a4_gemm_mx_planes(4, 4, 384, p, p, p, p, p, None) == W.WUSH_E_SHAPE
    assert L.wush_w4a4_gemm_mx_planes(4, 4, 512, None, p, p, p, p, None) == W.WUSH_E_ARG


def test_block_moments_dev_checks_and_workspace_size():
    L = W.lib
    # 300 tokens: 2 chunks of up to 256; 5000: 20; 20000: capped at 64
    assert L.wush_block_moments_dev_ws_bytes(32, 300, 128) == 2 * 128 * 32 * 8
    assert L.wush_block_moments_dev_ws_bytes(16, 5000, 64) == 20 * 64 * 16 * 8
    assert L.wush_block_moments_dev_ws_bytes(32, 20000, 64) == 64 * 64 * 32 * 8
    assert L.wush_block_moments_dev_ws_bytes(24, 300, 96) == 0
    assert L.wush_block_moments_dev(24, 0, 10, 96, None, None, None, 0, None) == W.WUSH_E_SHAPE
    assert L.wush_block_moments_dev(32, 0, 0, 64, None, None, None, 0, None) == W.WUSH_E_SHAPE
    assert L.wush_block_moments_dev(32, 0, 10, 64, None, None, None, 0, None) == W.WUSH_E_ARG


def _device_asm(src):
    import subprocess
    from aware_block_transforms_amd import build as B
    r = subprocess.run([B.HIPCC, *B.HIP_FLAGS, *B.HIP_EXTRA.get(src, []), "--cuda-device-only", "-S", "-o", "-",
                        os.path.join(B.CSRC, src)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def _kernel_code(asm, name):
    """Instructions (and labels) of the kernel whose symbol contains `name`."""
    import re
    out, on = [], False
    for line in asm.splitlines():
        if not on and re.match(r"^_Z\S*:", line) and name in line.split(":")[0]:
            on = True
            continue
        if on:
            t = line.split(";")[0].strip()
            if t.startswith("s_endpgm"):
                break
            if not t or t.startswith((".", "//")) and not re.match(r"^\.LBB\w*:", t):
                continue
            out.append(t)
    return out


def _vregs(tok):
    """VGPR numbers named by an operand token: v7 -> {7}, v[4:7] -> {4..7}."""
    import re
    m = re.fullmatch(r"v(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _asm_mfma_hazards(code, gap=3, acc_wait=19):
    """Hazards of inline-asm MFMAs in compiled code (list of instructions and labels).

    Returns the violations: a vector-ALU instruction writing an MFMA's A or B
    operand with fewer than `gap` wait states between it and the MFMA (s_nop N counts N + 1; branches
    into a label are followed back to their source, so a loop's back edge is
    covered), and fewer than `acc_wait` wait states between the last MFMA and
    the first instruction that reads an AGPR.
    """
    import re
    preds = {}
    for i, l in enumerate(code):
        m = re.match(r"s_c?branch\w*\s+(\.LBB\w+)", l)
        if m:
            preds.setdefault(m.group(1), []).append(i)

    def wait_states(ins):
        m = re.match(r"s_nop\s+(\d+)", ins)
        return int(m.group(1)) + 1 if m else 1

    def before(i, need, seen):
        found, k, left = [], i - 1, need
        while left > 0 and k >= 0:
            ins = code[k]
            if ins.endswith(":"):
                for b in preds.get(ins[:-1], []):
                    if (b, left) not in seen:
                        seen.add((b, left))
                        found += before(b + 1, left, seen)
                k -= 1
                continue
            found.append(ins)
            left -= wait_states(ins)
            k -= 1
        return found

    bad = []
    mfmas = [i for i, l in enumerate(code) if l.startswith("v_mfma")]
    for i in mfmas:
        ops = [t.strip() for t in code[i].split(None, 1)[1].split(",")]
        srcs = _vregs(ops[1]) | _vregs(ops[2])
        for prev in before(i, gap, set()):
            if prev.startswith("v_") and not prev.startswith("v_mfma") and " " in prev:
                if _vregs(prev.split(None, 1)[1].split(",")[0].strip()) & srcs:
                    bad.append((code[i], prev))
    if mfmas:
        ws = 0
        for ins in code[mfmas[-1] + 1:]:
            if not ins.endswith(":") and re.search(r"\ba(\d+|\[\d+:\d+\])", ins.split(None, 1)[-1]):
                break
            ws += 0 if ins.endswith(":") else wait_states(ins)
        if ws < acc_wait:
            bad.append(("accumulators read after", ws))
    return bad


def test_asm_mfma_hazard_checker_on_planted_cases():
    mfma = "v_mfma_f32_32x32x16_f16 a[0:15], v[4:7], v[8:11], a[0:15]"
    tail = ["s_nop 15", "s_nop 3", "v_accvgpr_read_b32 v0, a0"]
    assert _asm_mfma_hazards(["v_mov_b32_e32 v5, 0", mfma] + tail)                  # no wait state between
    assert _asm_mfma_hazards(["v_mov_b32_e32 v9, 0", "s_nop 1", mfma] + tail)       # 2 wait states between
    assert not _asm_mfma_hazards(["v_mov_b32_e32 v9, 0", "s_nop 2", mfma] + tail)   # 3 wait states between
    assert not _asm_mfma_hazards(["v_mov_b32_e32 v12, 0", mfma] + tail)             # not an operand
    # written at the end of the loop body, read by the MFMA at the loop head
    loop = [".LBB0_1:", mfma, "s_nop 7", "v_mov_b32_e32 v6, 1", "s_cbranch_scc1 .LBB0_1"] + tail
    assert _asm_mfma_hazards(loop)
    # accumulators read too early
    assert _asm_mfma_hazards(["s_nop 7", mfma, "s_nop 3", "v_accvgpr_read_b32 v0, a0"])


def test_asm_mfma_operands_are_written_early():
    """The NVFP4 matmul issues its MFMAs as inline asm, which the compiler's
    hazard recognizer does not see.  In the compiled kernel no vector-ALU
    instruction may write an MFMA's A or B operand with fewer than three wait
    states between the write and the MFMA, and the accumulators are read only after at least 19
    wait states past the last MFMA (see _asm_mfma_hazards)."""
    code = _kernel_code(_device_asm("gemm_nvfp4.hip"), "gemm_nvfp4_lds")
    assert sum(1 for l in code if l.startswith("v_mfma")) >= 64
    assert _asm_mfma_hazards(code) == []


def _loop_bodies(code):
    """Instruction lists of the innermost loops (a label followed later by a
    backward branch to it, with no other label in between)."""
    import re
    loops = []
    for i, line in enumerate(code):
        m = re.match(r"^(\.LBB\w*):$", line)
        if not m:
            continue
        body = []
        for l in code[i + 1:]:
            if re.match(r"^\.LBB\w*:$", l):
                body = None
                break
            body.append(l)
            if l.startswith("s_cbranch") and l.split()[-1] == m.group(1):
                break
        else:
            body = None
        if body:
            loops.append(body)
    return loops


def test_transform_loop_waits_cover_one_unit():
    """The streaming transform kernel keeps kDepth = 4 units of x loads in
    flight, with each unit's stores between them; its prologue issues matching
    stores into a zero-size resource so that every load wait in the loop waits
    for one unit's loads only.  Loads and stores retire through one in-order
    counter, and `s_waitcnt vmcnt(n)` leaves the n most recent operations in
    flight.  Replaying the compiled loop of the MXFP4 plane-order kernel (bf16,
    merged stores) in steady state, every wait must therefore leave the loads
    of the other three units (2 each) in flight; a regression to the
    prologue-only state shows as smaller counts at the loop's first units."""
    import re
    asm = _device_asm("transform_quant.hip")
    for stream in (0, 1):   # default and non-temporal x loads (x larger than the Infinity Cache)
        code = _kernel_code(asm, "tq_dense_kernelILi32ELi5ELb1ELb1ELb%dE" % stream)
        _check_loop_waits(code, stream)


def _check_loop_waits(code, stream):
    import re
    loops = [b for b in _loop_bodies(code) if sum(1 for l in b if l.startswith("v_mfma")) >= 64]
    assert len(loops) == 1, len(loops)
    x_loads = [l for l in loops[0] if l.startswith("buffer_load_dwordx4")]
    assert x_loads and all(l.rstrip().endswith(" nt") == bool(stream) for l in x_loads), x_loads
    ops = []
    for l in loops[0]:
        m = re.search(r"vmcnt\((\d+)\)", l)
        if m:
            ops.append(int(m.group(1)))
        elif l.startswith("buffer_load"):
            ops.append("L")
        elif l.startswith("buffer_store"):
            ops.append("S")
    assert ops.count("L") == 8 and ops.count("S") == 8, ops
    waits = [o for o in ops if isinstance(o, int)]
    assert waits, ops
    issued, in_flight = [], []
    for rep in range(3):                     # the first copy only fills the history
        for o in ops:
            if isinstance(o, int):
                if rep:
                    in_flight.append(issued[-o:].count("L") if o else 0)
            else:
                issued.append(o)
    assert min(in_flight) >= 6, (waits, in_flight)
