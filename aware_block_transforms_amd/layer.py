"""Allocation helpers around the libwush calls for one quantized linear layer.

``W4A4Layer`` holds the device-resident pieces of one layer (transform
matrices, packed weight codes and scales) and exposes the online path
(transform + quantize activations, then the W4A4 matmul) as two library
calls.  Tensors come from torch's caching allocator; every byte of
arithmetic runs inside libwush.so.
"""

import numpy as np
import torch

from . import _lib as W


def codes_shape(rows, d_in):
    return (rows, d_in // 2)


def scales_dtype(fmt):
    return torch.int16 if fmt == "int4" else torch.uint8


class W4A4Layer:
    """Weights Wt [d_out][d_in] (nn.Linear layout) quantized with a per-block transform."""

    def __init__(self, fmt, kind, Wt, Sx=None, device="cuda", build_host=True, Tx=None, Tw=None):
        """Wt: host float32 [d_out][d_in]; Sx: host float32 [d_in/bs][bs][bs] moments.

        The transform pair is built on the host by wush_build_transforms unless
        Tx / Tw (host float32 [nblk][bs][bs]) are given.
        """
        self.fmt, self.kind = fmt, kind
        self.bs = W.BLOCK[fmt]
        Wt = np.ascontiguousarray(Wt, dtype=np.float32)
        self.d_out, self.d_in = Wt.shape
        nblk = self.d_in // self.bs
        if Tx is None:
            Tx = np.empty((nblk, self.bs, self.bs), np.float32)
            Tw = np.empty_like(Tx)
            if kind in ("wus", "wush") and Sx is None:
                raise ValueError("WUS/WUSH need activation moments Sx")
            W.wush_build_transforms(kind, self.bs, Wt, None if Sx is None else np.ascontiguousarray(Sx, np.float32),
                                    Tx, Tw)
        self.Tx_host, self.Tw_host = Tx, Tw
        self.identity = kind == "identity"
        self.Tx = None if self.identity else torch.from_numpy(np.ascontiguousarray(Tx)).to(device)
        self.Tw = None if self.identity else torch.from_numpy(np.ascontiguousarray(Tw)).to(device)
        Wd = torch.from_numpy(Wt).to(device)
        self.w_codes = torch.empty(codes_shape(self.d_out, self.d_in), dtype=torch.uint8, device=device)
        self.w_scales = torch.empty((self.d_out, nblk), dtype=scales_dtype(fmt), device=device)
        self.w_g = W.wush_pack_weights(fmt, Wd, self.Tw, self.w_codes, self.w_scales)
        del Wd
        self.x_g = 1.0
        self._ws = None   # GEMM workspace, grown on demand

    def calibrate(self, X):
        """NVFP4 only: per-tensor activation scale from calibration activations (device tensor)."""
        if self.fmt == "nvfp4":
            self.x_g = W.wush_nvfp4_global_scale(X, self.Tx)
        return self.x_g

    def alloc_activation_codes(self, n, device="cuda"):
        nblk = self.d_in // self.bs
        return (torch.empty(codes_shape(n, self.d_in), dtype=torch.uint8, device=device),
                torch.empty((n, nblk), dtype=scales_dtype(self.fmt), device=device))

    def quantize(self, X, codes, scales):
        W.wush_transform_quant(self.fmt, X, self.Tx, codes, scales, g=self.x_g)

    def matmul(self, codes, scales, Y):
        n = codes.shape[0]
        need = W.wush_w4a4_gemm_ws_bytes(self.fmt, n, self.d_out, self.d_in)
        if need and (self._ws is None or self._ws.numel() < need or self._ws.device != codes.device):
            self._ws = torch.empty(need, dtype=torch.uint8, device=codes.device)
        W.wush_w4a4_gemm(self.fmt, codes, scales, self.w_codes, self.w_scales, Y, a_g=self.x_g, b_g=self.w_g,
                         ws=self._ws if need else None)

    def forward(self, X, out=None):
        n = X.shape[0]
        codes, scales = self.alloc_activation_codes(n, X.device)
        self.quantize(X, codes, scales)
        Y = out if out is not None else torch.empty((n, self.d_out), dtype=torch.float32, device=X.device)
        self.matmul(codes, scales, Y)
        return Y
