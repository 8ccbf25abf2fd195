"""wush_w4a4_gemm_noalloc: the matmul with its scratch in a fixed device array.

Checked against wush_w4a4_gemm (caller workspace) on the same operands, two
calls in a row with the second on a smaller problem, for every format: both
entry points run the same kernels, so Y must be bit-identical, and within the
matmul tolerance of the oracle.
"""

import numpy as np
import pytest
import torch

import aware_block_transforms_amd as W
from oracle import quant, gemm as og
from gpu_util import DEV, to_dev, host, gemm_close

pytestmark = pytest.mark.gpu


def _operands(fmt, M, N, K, seed):
    rng = np.random.default_rng([seed, M, N, K])
    A = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1)))).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ga = gb = None
    if fmt == "nvfp4":
        ga, gb = quant.nvfp4_tensor_scale(A), quant.nvfp4_tensor_scale(B)
    ca, sa = quant.transform_quant(fmt, None, A, g=ga, identity=True)
    cb, sb = quant.transform_quant(fmt, None, B, g=gb, identity=True)
    return ca, sa, cb, sb, ga, gb


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_noalloc_matches_workspace_call_twice(fmt):
    # the second call is smaller, so stale planes of the first would show up
    for (M, N, K), seed in (((600, 520, 1024), 1), ((130, 260, 512), 2)):
        ca, sa, cb, sb, ga, gb = _operands(fmt, M, N, K, seed)
        args = (to_dev(ca), to_dev(sa), to_dev(cb), to_dev(sb))
        need = W.wush_w4a4_gemm_ws_bytes(fmt, M, N, K)
        assert 0 < need <= W.wush_w4a4_gemm_noalloc_max_ws_bytes()
        ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
        Y_ws = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
        Y_na = torch.full((M, N), np.nan, dtype=torch.float32, device=DEV)
        W.wush_w4a4_gemm(fmt, *args, Y_ws, a_g=ga or 1.0, b_g=gb or 1.0, ws=ws)
        W.wush_w4a4_gemm_noalloc(fmt, *args, Y_na, a_g=ga or 1.0, b_g=gb or 1.0)
        torch.cuda.synchronize()
        assert torch.equal(Y_ws, Y_na), (fmt, M, N, K)
        ok, worst = gemm_close(host(Y_na), og.w4a4_gemm(fmt, ca, sa, cb, sb, ga, gb))
        assert ok, (fmt, M, N, K, worst)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    cap = W.wush_w4a4_gemm_noalloc_max_ws_bytes()
    assert cap == 16 << 20
    # MXFP4 of both Qwen3-14B projections at 16384 tokens fits
    assert W.wush_w4a4_gemm_ws_bytes("mxfp4", 16384, 17408, 5120) <= cap
    assert W.wush_w4a4_gemm_ws_bytes("mxfp4", 16384, 5120, 17408) <= cap
    # a shape needing more is refused before anything is launched
    M, N, K = 16384, 5120, 17408
    assert W.wush_w4a4_gemm_ws_bytes("nvfp4", M, N, K) > cap
    st = W.lib.wush_w4a4_gemm_noalloc(1, M, N, K, 16, 16, 1.0, 16, 16, 1.0, 16, None)
    assert st == W.WUSH_E_SHAPE
    assert b"scratch" in W.lib.wush_last_error()
