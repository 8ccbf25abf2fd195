"""ctypes binding of libwush (argument marshalling only).

Every function here has the name of the C entry point it wraps and only
converts arguments (ints, floats, device pointers from torch tensors, the
current HIP stream) and turns a non-OK status into an exception.  All
computation happens inside libwush.so.  Importing this module fails loudly
when the library has not been built: there is no fallback path.
"""

import ctypes
import os

# torch ships its own HIP runtime.  Loading libwush.so first would map the
# system HIP/HSA runtime as well, and two runtimes in one process do not see
# each other's device state ("no ROCm-capable device" on launch, crashes in
# later copies).  Importing torch first makes libwush bind to the runtime torch
# already loaded (same soname).
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwush.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libwush.so not found at {LIB_PATH}; build it with "
        "`python -m aware_block_transforms_amd.build` (no CPU fallback exists)")

lib = ctypes.CDLL(LIB_PATH)

# enums (must match include/wush.h)
WUSH_OK, WUSH_E_ARG, WUSH_E_SHAPE, WUSH_E_NUMERIC, WUSH_E_HIP, WUSH_E_UNSUPPORTED = range(6)
FORMATS = {"mxfp4": 0, "nvfp4": 1, "int4": 2}
KINDS = {"identity": 0, "hadamard": 1, "wus": 2, "wush": 3}
DTYPES = {"f32": 0, "bf16": 1}
BLOCK = {"mxfp4": 32, "nvfp4": 16, "int4": 32}

_i, _f, _p, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_fp = ctypes.POINTER(ctypes.c_float)

_SIGS = {
    "wush_format_block": ([_i], _i),
    "wush_block_moments": ([_i, _i, _i, _p, _p], _i),
    "wush_build_transforms": ([_i, _i, _i, _i, _p, _p, _p, _p], _i),
    "wush_transform_quant": ([_i, _i, _i, _i, _p, _p, _f, _p, _p, _p], _i),
    "wush_transform_apply": ([_i, _i, _i, _i, _p, _p, _p, _p], _i),
    "wush_build_shared": ([_i, _i, _i, _i, _p, _p, _i, _p, _p, _p], _i),
    "wush_mxfp4_planes_bytes": ([_i, _i], _sz),
    "wush_build_transforms_dev_ws_bytes": ([_i, _i], _sz),
    "wush_build_transforms_dev": ([_i, _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p], _i),
    "wush_mxfp4_scale_planes": ([_i, _i, _p, _p, _p], _i),
    "wush_transform_quant_mx_planes": ([_i, _i, _i, _p, _p, _p, _p, _p], _i),
    "wush_w4a4_gemm_mx_planes": ([_i, _i, _i, _p, _p, _p, _p, _p, _p], _i),
    "wush_transform_quant_shared": ([_i, _i, _i, _i, _p, _p, _i, _p, _f, _p, _p, _p], _i),
    "wush_nvfp4_global_scale_shared": ([_i, _i, _i, _p, _p, _i, _p, _p, _p], _i),
    "wush_pack_weights_shared": ([_i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _p], _i),
    "wush_nvfp4_global_scale": ([_i, _i, _i, _p, _p, _fp, _p], _i),
    "wush_pack_weights": ([_i, _i, _i, _p, _p, _p, _p, _fp, _p], _i),
    "wush_build_hd": ([_i, _i, _i, _p, _p, _p, _p], _i),
    "wush_block_moments_dev_ws_bytes": ([_i, _i, _i], _sz),
    "wush_block_moments_dev": ([_i, _i, _i, _i, _p, _p, _p, _sz, _p], _i),
    "wush_transform_quant_hd": ([_i, _i, _i, _i, _p, _p, _f, _p, _p, _p], _i),
    "wush_nvfp4_global_scale_hd": ([_i, _i, _i, _p, _p, _fp, _p], _i),
    "wush_pack_weights_hd": ([_i, _i, _i, _p, _p, _p, _p, _fp, _p], _i),
    "wush_w4a4_gemm_ws_bytes": ([_i, _i, _i, _i], _sz),
    "wush_w4a4_gemm": ([_i, _i, _i, _i, _p, _p, _f, _p, _p, _f, _p, _p, _sz, _p], _i),
    "wush_w4a4_gemm_noalloc_max_ws_bytes": ([], _sz),
    "wush_w4a4_gemm_noalloc": ([_i, _i, _i, _i, _p, _p, _f, _p, _p, _f, _p, _p], _i),
    "wush_layer_loss": ([_i, _i, _p, _p, _p, _p, _p], _i),
    "wush_loss_ws_bytes": ([_i, _i], _sz),
    "wush_had256_packed_bytes": ([_i, _i], _sz),
    "wush_had256_pack_weights": ([_i, _i, _p, _p, _p], _i),
    "wush_had256_gemv_ws_bytes": ([_i, _i], _sz),
    "wush_had256_gemv": ([_i, _i, _i, _p, _p, _p, _p, _sz, _p], _i),
    "wush_had256_rotate": ([_i, _i, _p, _p, _p], _i),
    "wush_status_string": ([_i], ctypes.c_char_p),
    "wush_last_error": ([], ctypes.c_char_p),
    "wush_version": ([], ctypes.c_char_p),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret

EXPORTED = tuple(_SIGS)


class WushError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = lib.wush_last_error().decode()
        super().__init__(f"{where}: {lib.wush_status_string(status).decode()} ({status}): {detail}")


def _check(status, where):
    if status != WUSH_OK:
        raise WushError(status, where)


def _ptr(t):
    """Raw address of a torch tensor / numpy array (or None)."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


# ----------------------------------------------------------------------------- host calls


def wush_block_moments(bs, X, Sx):
    """X: host float32 [n][d_in] (numpy or CPU tensor), Sx: host float32 [d_in/bs][bs][bs] out."""
    n, d_in = X.shape
    _check(lib.wush_block_moments(bs, n, d_in, _ptr(X), _ptr(Sx)), "wush_block_moments")


def wush_build_transforms(kind, bs, W, Sx, Tx, Tw):
    """Host arrays: W [d_out][d_in] f32, Sx [nblk][bs][bs] f32 (or None), Tx/Tw out."""
    k = KINDS[kind] if isinstance(kind, str) else int(kind)
    d_out, d_in = (W.shape if W is not None else (0, Tx.shape[0] * bs))
    _check(lib.wush_build_transforms(k, bs, d_in, d_out, _ptr(W), _ptr(Sx), _ptr(Tx), _ptr(Tw)),
           "wush_build_transforms")


def wush_build_hd(bs, W, Sx, dx, dw):
    """Host arrays: W [d_out][d_in] f32, Sx [nblk][bs][bs] f32; dx, dw out [d_in] f32."""
    d_out, d_in = W.shape
    _check(lib.wush_build_hd(bs, d_in, d_out, _ptr(W), _ptr(Sx), _ptr(dx), _ptr(dw)), "wush_build_hd")


# ----------------------------------------------------------------------------- device calls


def wush_transform_quant(fmt, X, Tx, codes, scales, g=0.0, stream=None):
    """X: device [n][d_in] float32 or bfloat16; Tx: device [nblk][bs][bs] f32 or None (identity)."""
    import torch
    n, d_in = X.shape
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("X must be float32 or bfloat16")
    _check(lib.wush_transform_quant(_fmt(fmt), xdt, n, d_in, _ptr(X), _ptr(Tx), float(g), _ptr(codes),
                                    _ptr(scales), _stream(stream)), "wush_transform_quant")


def wush_transform_apply(X, Tx, Y, stream=None):
    """Y = T x per block (fp32, the transform wush_transform_quant quantizes).  Tx: [nblk][bs][bs]."""
    import torch
    n, d_in = X.shape
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("X must be float32 or bfloat16")
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    _check(lib.wush_transform_apply(xdt, Tx.shape[-1], n, d_in, _ptr(X), _ptr(Tx), _ptr(Y), _stream(stream)),
           "wush_transform_apply")


def wush_build_shared(kind, W, Sx, bs, group, ngroups):
    """Host numpy: per-group (Tx, Tw) [ngroups][bs][bs] float32 from the groups' summed moments."""
    import numpy as np
    W = np.ascontiguousarray(W, dtype=np.float32)
    d_out, d_in = W.shape
    group = np.ascontiguousarray(group, dtype=np.int32)
    Sx = None if Sx is None else np.ascontiguousarray(Sx, dtype=np.float32)
    Tx = np.empty((ngroups, bs, bs), dtype=np.float32)
    Tw = np.empty_like(Tx)
    _check(lib.wush_build_shared(KINDS[kind], bs, d_in, d_out, W.ctypes.data,
                                 None if Sx is None else Sx.ctypes.data, int(ngroups), group.ctypes.data,
                                 Tx.ctypes.data, Tw.ctypes.data), "wush_build_shared")
    return Tx, Tw


def wush_transform_quant_shared(fmt, X, Tx, group, codes, scales, g=0.0, stream=None):
    """X: device [n][d_in] f32/bf16; Tx: device [ngroups][bs][bs] f32; group: device [nblk] int32."""
    import torch
    n, d_in = X.shape
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("X must be float32 or bfloat16")
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    _check(lib.wush_transform_quant_shared(_fmt(fmt), xdt, n, d_in, _ptr(X), _ptr(Tx), Tx.shape[0], _ptr(group),
                                           float(g), _ptr(codes), _ptr(scales), _stream(stream)),
           "wush_transform_quant_shared")


def wush_nvfp4_global_scale_shared(X, Tx, group, stream=None):
    import torch
    n, d_in = X.shape
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    g = ctypes.c_float(0.0)
    _check(lib.wush_nvfp4_global_scale_shared(xdt, n, d_in, _ptr(X), _ptr(Tx), Tx.shape[0], _ptr(group),
                                              ctypes.byref(g), _stream(stream)), "wush_nvfp4_global_scale_shared")
    return g.value


def wush_pack_weights_shared(fmt, W, Tw, group, codes, scales, stream=None):
    """W: device [d_out][d_in] f32.  Returns the NVFP4 tensor scale (1.0 for other formats)."""
    d_out, d_in = W.shape
    g = ctypes.c_float(0.0)
    _check(lib.wush_pack_weights_shared(_fmt(fmt), d_out, d_in, _ptr(W), _ptr(Tw), Tw.shape[0], _ptr(group),
                                        _ptr(codes), _ptr(scales), ctypes.byref(g), _stream(stream)),
           "wush_pack_weights_shared")
    return g.value


def wush_build_transforms_dev_ws_bytes(bs, d_in):
    return lib.wush_build_transforms_dev_ws_bytes(bs, d_in)


def wush_build_transforms_dev(kind, bs, W, Sx, Tx, Tw, ws=None, stream=None):
    """Device tensors: W [d_out][d_in] f32, Sx [nblk][bs][bs] f32 -> Tx, Tw [nblk][bs][bs] f32 (synchronises)."""
    import torch
    d_out, d_in = W.shape
    need = lib.wush_build_transforms_dev_ws_bytes(bs, d_in)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=Tx.device)
    _check(lib.wush_build_transforms_dev(KINDS[kind], bs, d_in, d_out, _ptr(W), _ptr(Sx), _ptr(Tx), _ptr(Tw), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)), "wush_build_transforms_dev")


def wush_mxfp4_planes_bytes(rows, K):
    return lib.wush_mxfp4_planes_bytes(rows, K)


def wush_mxfp4_scale_planes(scales, planes, K, stream=None):
    """scales: device [rows][K/32] uint8 (row-major) -> planes: device uint8 of wush_mxfp4_planes_bytes."""
    _check(lib.wush_mxfp4_scale_planes(scales.shape[0], K, _ptr(scales), _ptr(planes), _stream(stream)),
           "wush_mxfp4_scale_planes")


def wush_transform_quant_mx_planes(X, Tx, codes, planes, stream=None):
    import torch
    n, d_in = X.shape
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("X must be float32 or bfloat16")
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    _check(lib.wush_transform_quant_mx_planes(xdt, n, d_in, _ptr(X), _ptr(Tx), _ptr(codes), _ptr(planes),
                                              _stream(stream)), "wush_transform_quant_mx_planes")


def wush_w4a4_gemm_mx_planes(a_codes, a_planes, b_codes, b_planes, Y, stream=None):
    M, N = Y.shape
    K = a_codes.shape[1] * 2
    _check(lib.wush_w4a4_gemm_mx_planes(M, N, K, _ptr(a_codes), _ptr(a_planes), _ptr(b_codes), _ptr(b_planes),
                                        _ptr(Y), _stream(stream)), "wush_w4a4_gemm_mx_planes")


def wush_nvfp4_global_scale(X, Tx, stream=None):
    import torch
    n, d_in = X.shape
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    g = ctypes.c_float(0.0)
    _check(lib.wush_nvfp4_global_scale(xdt, n, d_in, _ptr(X), _ptr(Tx), ctypes.byref(g), _stream(stream)),
           "wush_nvfp4_global_scale")
    return g.value


def wush_pack_weights(fmt, W, Tw, codes, scales, stream=None):
    """W: device [d_out][d_in] f32.  Returns the NVFP4 tensor scale (1.0 for other formats)."""
    d_out, d_in = W.shape
    g = ctypes.c_float(0.0)
    _check(lib.wush_pack_weights(_fmt(fmt), d_out, d_in, _ptr(W), _ptr(Tw), _ptr(codes), _ptr(scales),
                                 ctypes.byref(g), _stream(stream)), "wush_pack_weights")
    return g.value


def wush_block_moments_dev_ws_bytes(bs, n, d_in):
    return lib.wush_block_moments_dev_ws_bytes(bs, n, d_in)


def wush_block_moments_dev(bs, X, Sx, ws=None, stream=None):
    """X: device [n][d_in] float32 or bfloat16; Sx: device out [d_in/bs][bs][bs] float32."""
    import torch
    n, d_in = X.shape
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("X must be float32 or bfloat16")
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    wp, wb = _ws(ws)
    _check(lib.wush_block_moments_dev(bs, xdt, n, d_in, _ptr(X), _ptr(Sx), wp, wb, _stream(stream)),
           "wush_block_moments_dev")


def wush_transform_quant_hd(fmt, X, dx, codes, scales, g=0.0, stream=None):
    """Hadamard-diagonal variant; dx: device [d_in] f32 (from wush_build_hd)."""
    import torch
    n, d_in = X.shape
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("X must be float32 or bfloat16")
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    _check(lib.wush_transform_quant_hd(_fmt(fmt), xdt, n, d_in, _ptr(X), _ptr(dx), float(g), _ptr(codes),
                                       _ptr(scales), _stream(stream)), "wush_transform_quant_hd")


def wush_nvfp4_global_scale_hd(X, dx, stream=None):
    import torch
    n, d_in = X.shape
    xdt = DTYPES["bf16"] if X.dtype == torch.bfloat16 else DTYPES["f32"]
    g = ctypes.c_float(0.0)
    _check(lib.wush_nvfp4_global_scale_hd(xdt, n, d_in, _ptr(X), _ptr(dx), ctypes.byref(g), _stream(stream)),
           "wush_nvfp4_global_scale_hd")
    return g.value


def wush_pack_weights_hd(fmt, W, dw, codes, scales, stream=None):
    """W: device [d_out][d_in] f32, dw: device [d_in] f32.  Returns the NVFP4 tensor scale (1.0 otherwise)."""
    d_out, d_in = W.shape
    g = ctypes.c_float(0.0)
    _check(lib.wush_pack_weights_hd(_fmt(fmt), d_out, d_in, _ptr(W), _ptr(dw), _ptr(codes), _ptr(scales),
                                    ctypes.byref(g), _stream(stream)), "wush_pack_weights_hd")
    return g.value


def _ws(ws):
    """(pointer, bytes) of an optional device workspace tensor."""
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def wush_w4a4_gemm_ws_bytes(fmt, M, N, K):
    return lib.wush_w4a4_gemm_ws_bytes(_fmt(fmt), M, N, K)


def wush_w4a4_gemm(fmt, a_codes, a_scales, b_codes, b_scales, Y, a_g=1.0, b_g=1.0, ws=None, stream=None):
    M, N = Y.shape
    K = a_codes.shape[1] * 2
    wp, wb = _ws(ws)
    _check(lib.wush_w4a4_gemm(_fmt(fmt), M, N, K, _ptr(a_codes), _ptr(a_scales), float(a_g), _ptr(b_codes),
                              _ptr(b_scales), float(b_g), _ptr(Y), wp, wb, _stream(stream)), "wush_w4a4_gemm")


def wush_w4a4_gemm_noalloc_max_ws_bytes():
    return lib.wush_w4a4_gemm_noalloc_max_ws_bytes()


def wush_w4a4_gemm_noalloc(fmt, a_codes, a_scales, b_codes, b_scales, Y, a_g=1.0, b_g=1.0, stream=None):
    M, N = Y.shape
    K = a_codes.shape[1] * 2
    _check(lib.wush_w4a4_gemm_noalloc(_fmt(fmt), M, N, K, _ptr(a_codes), _ptr(a_scales), float(a_g), _ptr(b_codes),
                                      _ptr(b_scales), float(b_g), _ptr(Y), _stream(stream)), "wush_w4a4_gemm_noalloc")


def wush_loss_ws_bytes(M, N):
    return lib.wush_loss_ws_bytes(M, N)


def wush_layer_loss(Yhat, Yref, loss, ws, stream=None):
    M, N = Yhat.shape
    _check(lib.wush_layer_loss(M, N, _ptr(Yhat), _ptr(Yref), _ptr(loss), _ptr(ws), _stream(stream)),
           "wush_layer_loss")


def wush_had256_packed_bytes(d_out, d_in):
    return lib.wush_had256_packed_bytes(d_out, d_in)


def _packed_check(packed, d_out, d_in, name):
    need = lib.wush_had256_packed_bytes(d_out, d_in)
    if packed.numel() * packed.element_size() < need:
        raise ValueError("%s: packed buffer of %d bytes, need %d" % (name, packed.numel() * packed.element_size(), need))


def wush_had256_pack_weights(W, packed, stream=None):
    d_out, d_in = W.shape
    _packed_check(packed, d_out, d_in, "wush_had256_pack_weights")
    _check(lib.wush_had256_pack_weights(d_out, d_in, _ptr(W), _ptr(packed), _stream(stream)),
           "wush_had256_pack_weights")


def wush_had256_gemv_ws_bytes(batch, d_in):
    return lib.wush_had256_gemv_ws_bytes(batch, d_in)


def wush_had256_gemv(x, packed, y, ws=None, stream=None):
    batch, d_in = x.shape
    d_out = y.shape[1]
    _packed_check(packed, d_out, d_in, "wush_had256_gemv")
    wp, wb = _ws(ws)
    _check(lib.wush_had256_gemv(batch, d_out, d_in, _ptr(x), _ptr(packed), _ptr(y), wp, wb, _stream(stream)),
           "wush_had256_gemv")


def wush_had256_rotate(inp, out, stream=None):
    rows, d_in = inp.shape
    _check(lib.wush_had256_rotate(rows, d_in, _ptr(inp), _ptr(out), _stream(stream)), "wush_had256_rotate")


def wush_version():
    return lib.wush_version().decode()
