"""Seeded generators for the five evaluation workloads (no method arithmetic).

Every array comes from ``numpy.random.default_rng([config_id, stream])``:
stream 0 = weights, 1 = activations, 2 = outlier-channel indices, 3 = outlier
channel factors, 4 = weight-outlier positions, 5 = weight-outlier values.
bf16 storage is produced by a round-to-nearest-even cast (torch CPU).

Shapes follow the layers the WUSH article evaluates on (Qwen3-8B block 18,
Qwen3-14B; paragraph on experiments) and the ITQ3_S article's 256-vector
weight quantization; the real checkpoints are not available, so these seeded
tensors stand in for them.
"""

from dataclasses import dataclass, field

import numpy as np
import torch


def bf16_round(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(x):
    """bf16 bit patterns (uint16) of bf16-representable float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    d_in: int
    d_out: int
    n: int
    act: str          # activation model
    weight: str       # weight model
    dtype: str        # activation storage dtype: "f32" or "bf16"
    formats: tuple = ("mxfp4",)
    kinds: tuple = ("wush",)
    extra: dict = field(default_factory=dict)

    @property
    def flops(self):
        return 2.0 * self.n * self.d_out * self.d_in


CONFIGS = {
    # Single 256x256 layer, 128 tokens, fp32; MXFP4; identity / Hadamard / WUSH.
    "tiny": Workload(1, "tiny-256x256-n128", 256, 256, 128, "gauss_x50", "t3", "f32",
                     ("mxfp4",), ("identity", "hadamard", "wush")),
    # Qwen3-8B MLP up-projection 4096 -> 12288 at 4096 tokens, bf16, MXFP4, WUSH.
    "qwen3_8b_up": Workload(2, "qwen3-8b-up-4096x12288-n4096", 4096, 12288, 4096,
                            "gauss_logu", "gauss_t", "bf16"),
    # 4096x4096 square projection, 8192 tokens, fp32; 3 formats x 4 transforms.
    "square_sweep": Workload(3, "square-4096x4096-n8192", 4096, 4096, 8192, "gauss_x50", "t3",
                             "f32", ("mxfp4", "nvfp4", "int4"),
                             ("identity", "hadamard", "wus", "wush")),
    # Qwen3-14B up_proj 5120 -> 17408 and down_proj 17408 -> 5120 at 16384 tokens.
    "qwen3_14b_up": Workload(4, "qwen3-14b-up-5120x17408-n16384", 5120, 17408, 16384,
                             "gauss_logu", "gauss_t", "bf16"),
    "qwen3_14b_down": Workload(40, "qwen3-14b-down-17408x5120-n16384", 17408, 5120, 16384,
                               "laplace_x50", "gauss_t", "bf16"),
    # Hadamard-256 3-bit weight-only GEMV, 4096 -> 14336, batch 1 / 4 / 16.
    "had256": Workload(5, "had256-4096x14336", 4096, 14336, 16, "gauss", "gauss_t", "bf16",
                       (), (), {"batches": (1, 4, 16)}),
}


def _rng(cid, stream):
    return np.random.default_rng([cid, stream])


def make_weights(w: Workload, d_out=None, d_in=None):
    """Weights in nn.Linear layout Wt [d_out][d_in] (float32)."""
    d_out = d_out or w.d_out
    d_in = d_in or w.d_in
    r = _rng(w.cid, 0)
    if w.weight == "t3":
        # 0.02 * Student-t with 3 degrees of freedom
        W = 0.02 * r.standard_t(3, size=(d_out, d_in))
    elif w.weight == "gauss_t":
        # N(0, 0.02) plus Student-t(3) outliers (scale 0.02) added at 0.01% of entries
        W = r.normal(0.0, 0.02, size=(d_out, d_in))
        k = max(1, int(round(1e-4 * d_out * d_in)))
        pos = _rng(w.cid, 4).choice(d_out * d_in, size=k, replace=False)
        W.reshape(-1)[pos] += 0.02 * _rng(w.cid, 5).standard_t(3, size=k)
    else:
        raise ValueError(w.weight)
    return W.astype(np.float32)


def make_activations(w: Workload, n=None, d_in=None):
    """Activations token-major Xt [n][d_in] as float32 (bf16-rounded when the workload is bf16)."""
    n = n or w.n
    d_in = d_in or w.d_in
    r = _rng(w.cid, 1)
    if w.act == "gauss_x50":
        # N(0,1) with 4 seeded outlier channels scaled x50
        X = r.standard_normal((n, d_in), dtype=np.float32)
        ch = _rng(w.cid, 2).choice(d_in, size=4, replace=False)
        X[:, ch] *= 50.0
    elif w.act == "gauss_logu":
        # N(0,1) with 0.1% of channels scaled by log-uniform factors in [20, 100]
        X = r.standard_normal((n, d_in), dtype=np.float32)
        k = max(1, int(round(1e-3 * d_in)))
        ch = _rng(w.cid, 2).choice(d_in, size=k, replace=False)
        f = np.exp(_rng(w.cid, 3).uniform(np.log(20.0), np.log(100.0), size=k))
        X[:, ch] *= f.astype(np.float32)
    elif w.act == "laplace_x50":
        # heavy-tailed Laplace(0, 1) (stands in for the SiLU-gated down_proj input)
        # with 0.2% of channels scaled x50
        X = r.laplace(0.0, 1.0, size=(n, d_in)).astype(np.float32)
        k = max(1, int(round(2e-3 * d_in)))
        ch = _rng(w.cid, 2).choice(d_in, size=k, replace=False)
        X[:, ch] *= 50.0
    elif w.act == "gauss":
        X = r.standard_normal((n, d_in), dtype=np.float32)
    else:
        raise ValueError(w.act)
    X = X.astype(np.float32)
    if w.dtype == "bf16":
        X = bf16_round(X)
    return X


def random_case(seed, n, d_in, d_out, dtype="f32", outliers=4, scale=50.0):
    """Small seeded case for parity tests: (Wt, Xt)."""
    r = np.random.default_rng([1000 + seed, 0])
    W = (0.02 * r.standard_t(3, size=(d_out, d_in))).astype(np.float32)
    X = r.standard_normal((n, d_in), dtype=np.float32)
    if outliers:
        ch = r.choice(d_in, size=min(outliers, d_in), replace=False)
        X[:, ch] *= scale
    if dtype == "bf16":
        X = bf16_round(X)
    return W, X
