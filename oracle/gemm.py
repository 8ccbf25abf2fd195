"""Quantized GEMM and layer loss (test infrastructure only).

Source: "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization" (AI
Radio episode), "Problem Setup and Goal": the layer loss is the squared L2
norm of q(T_W W)^T q(T_X X) - W^T X normalised by d_out times the batch size
(the page's rendering of the normaliser is garbled; d_out * batch is the
reading used).  The W4A4 product itself is the "FP4 MatMul" the same episode
credits with the per-layer speedup over BF16.

Operands are decoded exactly to fp64 (every E2M1 / E8M0 / E4M3 / fp16 value
and every INT4 level is a dyadic rational that fp64 holds exactly) and the
product is accumulated in fp64 with numpy's matmul.
"""

import numpy as np

from .fp import e2m1_value, e8m0_value, e4m3_value, f16_value
from .quant import unpack_nibbles


def decode(fmt, codes, scales, g=None):
    """Dequantize [rows][K/2] codes and their block scales to fp64 [rows][K]."""
    c = unpack_nibbles(codes)
    rows, K = c.shape
    if fmt == "mxfp4":
        v = e2m1_value(c).reshape(rows, K // 32, 32) * e8m0_value(scales)[..., None]
    elif fmt == "nvfp4":
        v = e2m1_value(c).reshape(rows, K // 16, 16) * e4m3_value(scales)[..., None]
        v = v * np.float64(np.float32(g))
    elif fmt == "int4":
        q = c.astype(np.int64)
        q = np.where(q >= 8, q - 16, q).astype(np.float64)
        v = q.reshape(rows, K // 32, 32) * f16_value(scales)[..., None]
    else:
        raise ValueError(fmt)
    return v.reshape(rows, K)


def w4a4_gemm(fmt, a_codes, a_scales, b_codes, b_scales, a_g=None, b_g=None):
    """Y[M][N] = dec(A) dec(B)^T in fp64.  A: activations [M][K], B: weights [N][K]."""
    A = decode(fmt, a_codes, a_scales, a_g)
    B = decode(fmt, b_codes, b_scales, b_g)
    return A @ B.T


def w4a4_gemm_rows(fmt, rows, a_codes, a_scales, b_codes, b_scales, a_g=None, b_g=None):
    """Only the listed output rows (for sampled checks of large problems)."""
    A = decode(fmt, a_codes[rows], a_scales[rows], a_g)
    B = decode(fmt, b_codes, b_scales, b_g)
    return A @ B.T


def reference_output(Wt, Xt):
    """Unquantized layer output W^T X in fp64, token-major [n][d_out]."""
    return np.asarray(Xt, dtype=np.float64) @ np.asarray(Wt, dtype=np.float64).T


def layer_loss(Yhat, Yref):
    """sum((Yhat - Yref)^2) / (d_out * n) in fp64."""
    Yhat = np.asarray(Yhat, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    return float(np.sum((Yhat - Yref) ** 2) / Yhat.size)
