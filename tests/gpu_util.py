"""Helpers shared by the GPU tests (marshalling only; no method arithmetic)."""

import numpy as np
import torch

from synth.gen import bf16_bits

DEV = "cuda"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x_dev(X, dtype):
    """Host float32 activations -> device tensor of the storage dtype (bf16 is exact: X is bf16-representable)."""
    if dtype == "bf16":
        bits = bf16_bits(X).view(np.int16)
        return to_dev(bits).view(torch.bfloat16)
    return to_dev(X.astype(np.float32))


def host(t):
    return t.detach().cpu().numpy()


def scales_np(t, fmt):
    a = host(t)
    return a.view(np.uint16) if fmt == "int4" else a.view(np.uint8)


def gemm_close(Y, ref, rel=1e-3):
    """Per-element criterion |Y - ref| <= rel * max(|ref|, rms(ref))."""
    Y = np.asarray(Y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    tol = rel * np.maximum(np.abs(ref), rms)
    bad = np.abs(Y - ref) > tol
    return (not bad.any()), float(np.max(np.abs(Y - ref) / np.maximum(tol, 1e-300))) if ref.size else 0.0
