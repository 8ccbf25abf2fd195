"""Per-block transform then block quantization (test infrastructure only).

Source: "WUSH" news article (chain.bitekongjian.com), paragraph on
experiments: MXFP4, NVFP4 and INT4 layer loss with the transform applied to
both weights and activations; paragraph on deployment: the activation
transform is applied online, one block-diagonal matrix per block.  "WUSH:
Near-Optimal Adaptive Transforms for LLM Quantization", "The gist": the
transform and the quantizer run fused on the GPU.

Pinned arithmetic (the pages leave it open; codes depend on every bit):

* transform:  y_i = fma chain over k = 0..bs-1 ascending, starting from +0:
              acc = fmaf(T[i][k], x[k], acc); identity is a bit-exact copy.
* MXFP4 (32): a = max|y|; e = clamp(floor(log2 a) - 2, -127, 127) (a = 0 ->
              -127); scale byte e + 127; code_i = E2M1(y_i * 2**-e); NaN/Inf
              block -> scale 0xFF, codes 0.
* NVFP4 (16): d = f32(6 g); s = f32(a / d); s8 = E4M3(min(s, 448));
              s_eff = f32(dec(s8) g); s_eff == 0 -> codes 0; r = f32(1/s_eff);
              code_i = E2M1(f32(y_i r)); NaN/Inf block -> scale 0x7F, codes 0.
* INT4  (32): s16 = fp16(f32(a / 7)); s16 == 0 -> codes 0; r = f32(1/f32(s16));
              q_i = clamp(rint_even(f32(y_i r)), -7, 7) stored as q & 0xF;
              NaN/Inf block -> scale 0x7E00, codes 0.
* packing:    byte j of a row holds code 2j in its low nibble, 2j+1 in its high.

The nibble order and the NVFP4 divisor 6 * 448 are format choices: the pages
fix neither.  Both are pinned by hand-derived bytes and scales in
tests/golden/packing.json, which do not pass through this module's unpack.
"""

import numpy as np

from .fp import fmaf, e2m1_code, e4m3_code, e4m3_value, f16_bits

FORMATS = ("mxfp4", "nvfp4", "int4")
BLOCK = {"mxfp4": 32, "nvfp4": 16, "int4": 32}


def apply_transform(T, Xt, identity=False):
    """y = T_b x_b per block and token, fp32 FMA chain (see module docstring).

    T: [nblk][bs][bs] float32; Xt: [n][d_in] float32.  Returns [n][d_in] float32.
    """
    Xt = np.asarray(Xt, dtype=np.float32)
    if identity:
        return Xt.copy()
    T = np.asarray(T, dtype=np.float32)
    nblk, bs, _ = T.shape
    n = Xt.shape[0]
    x = Xt.reshape(n, nblk, 1, bs)                    # [t][b][.][k]
    acc = np.zeros((n, nblk, bs), dtype=np.float32)  # +0
    for k in range(bs):
        acc = fmaf(T[None, :, :, k], x[:, :, 0, k][:, :, None], acc)
    return acc.reshape(n, nblk * bs)


def _blocks(y, bs):
    y = np.asarray(y, dtype=np.float32)
    n, d = y.shape
    return y.reshape(n, d // bs, bs)


def pack_nibbles(codes):
    """[n][d] codes (0..15) -> [n][d/2] bytes, low nibble = even index."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    n, h = packed.shape
    out = np.empty((n, 2 * h), dtype=np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


def quant_mxfp4(y):
    """MXFP4 quantization of already-transformed y [n][d] -> (codes [n][d/2], scales [n][d/32] u8)."""
    yb = _blocks(y, 32)
    a = np.max(np.abs(yb), axis=-1)                   # exact
    bad = ~np.isfinite(a)
    _, ex = np.frexp(np.where(bad | (a == 0), 1.0, a).astype(np.float64))
    e = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)   # floor(log2 a) = ex - 1
    e = np.where(a == 0, -127, e)
    scale = np.where(bad, 255, e + 127).astype(np.uint8)
    v = yb.astype(np.float64) * np.ldexp(1.0, -e)[..., None]   # exact power-of-two scaling
    codes = e2m1_code(v)
    codes = np.where(bad[..., None], 0, codes).astype(np.uint8)
    return pack_nibbles(codes.reshape(y.shape)), scale


def nvfp4_tensor_scale(y):
    """Default per-tensor scale g = f32(amax(y) / 2688) (2688 = 6 * 448)."""
    a = np.float32(np.max(np.abs(np.asarray(y, dtype=np.float32))))
    return np.float32(a / np.float32(2688.0))


def quant_nvfp4(y, g):
    """NVFP4 quantization of transformed y with per-tensor scale g -> (codes, scales u8 E4M3)."""
    g = np.float32(g)
    yb = _blocks(y, 16)
    a = np.max(np.abs(yb), axis=-1)
    bad = ~np.isfinite(a)
    d = np.float32(np.float32(6.0) * g)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        s = (np.where(bad, np.float32(0), a) / d).astype(np.float32)
        s = np.minimum(s, np.float32(448.0))
        s8 = e4m3_code(np.where(np.isfinite(s), s, 0.0))
        s_eff = (e4m3_value(s8).astype(np.float32) * g).astype(np.float32)
        r = (np.float32(1.0) / s_eff).astype(np.float32)
        v = (yb * r[..., None]).astype(np.float32)
    codes = e2m1_code(v)
    zero = (s_eff == 0) | bad
    codes = np.where(zero[..., None], 0, codes).astype(np.uint8)
    scale = np.where(bad, 0x7F, s8).astype(np.uint8)
    return pack_nibbles(codes.reshape(y.shape)), scale


def quant_int4(y):
    """INT4 (symmetric [-7, 7], fp16 scale per 32) of transformed y -> (codes, scales u16 fp16 bits)."""
    yb = _blocks(y, 32)
    a = np.max(np.abs(yb), axis=-1)
    bad = ~np.isfinite(a)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        sa = (np.where(bad, np.float32(0), a) / np.float32(7.0)).astype(np.float32)
        s16 = f16_bits(sa)
        s32 = s16.view(np.float16).astype(np.float32)
        r = (np.float32(1.0) / s32).astype(np.float32)
        t = (yb * r[..., None]).astype(np.float32)
    q = np.clip(np.rint(np.where(np.isfinite(t), t, 0.0)), -7, 7).astype(np.int64)
    q = np.where(((s32 == 0) | bad)[..., None], 0, q)
    codes = (q & 15).astype(np.uint8)
    scale = np.where(bad, 0x7E00, s16).astype(np.uint16)
    return pack_nibbles(codes.reshape(y.shape)), scale


def apply_hd(d, Xt, bs):
    """Hadamard-diagonal transform y = H_bs (d o x) per block and token, fp32.

    Pinned: v_k = f32(x_k * d_k) (a product, not fused into the butterflies),
    then butterfly stages h = 1, 2, ..., bs/2; in each stage every pair
    (j, j + h) with j in the lower half of a 2h-aligned group becomes
    (v_j + v_{j+h}, v_j - v_{j+h}), in fp32.
    d: [d_in] float32 (the Hadamard's 1/sqrt(bs) included); Xt: [n][d_in].
    """
    Xt = np.asarray(Xt, dtype=np.float32)
    n, d_in = Xt.shape
    v = (Xt * np.asarray(d, dtype=np.float32)[None, :]).astype(np.float32)
    h = 1
    while h < bs:
        w = v.reshape(n, d_in // (2 * h), 2, h)
        lo = w[:, :, 0, :].copy()
        hi = w[:, :, 1, :].copy()
        w[:, :, 0, :] = lo + hi
        w[:, :, 1, :] = lo - hi
        v = w.reshape(n, d_in)
        h *= 2
    return v


def quantize(fmt, y, g=None):
    """Block quantizer of an already transformed [n][d_in] fp32 array."""
    if fmt == "mxfp4":
        return quant_mxfp4(y)
    if fmt == "nvfp4":
        return quant_nvfp4(y, g)
    if fmt == "int4":
        return quant_int4(y)
    raise ValueError(fmt)


def transform_quant_hd(fmt, d, Xt, g=None):
    """Hadamard-diagonal activation step: apply_hd then the block quantizer."""
    return quantize(fmt, apply_hd(d, Xt, BLOCK[fmt]), g)


def transform_quant(fmt, T, Xt, g=None, identity=False):
    """Full activation-side step: transform then quantize.  Returns (codes, scales)."""
    y = apply_transform(T, Xt, identity=identity)
    if fmt == "mxfp4":
        return quant_mxfp4(y)
    if fmt == "nvfp4":
        return quant_nvfp4(y, g)
    if fmt == "int4":
        return quant_int4(y)
    raise ValueError(fmt)
