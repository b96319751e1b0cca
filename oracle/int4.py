"""Group-wise asymmetric INT4 quantization, packing and the fp64 W4A16 forward.

Test infrastructure only (see the package docstring).

Sources
  * Asymmetric quantization, "Quantization：模型量化" (xingyuwang.me),
    section 2 "Symmetric 与 Asymmetric Quantization": q = round(x/s) + z,
    x_hat = (q - z) s, followed by clipping to the integer range.
  * Per-group granularity, same page, section 3 "Per-group / Group-wise":
    an independent scale for every group of 32 / 64 / 128 weights.
  * Min-max range and the packed INT4 group format, "Lance-Quant" page
    (zingnex.cn), section "量化应用：网格搜索与分组策略" (awq_apply packs the
    weights group-wise into INT4; without activation data it falls back to
    min-max).
  * The quantized layer dequantizes in memory and is mathematically the
    original layer with W replaced by its dequantized value, "模型量化指南"
    (blog.yoooo.fun), section "共同约定".

Readings where the pages are silent (each listed in the design notes):
  * S = fl32(fl32(max - min) / 15); z = clamp(rne(fl32(-min / S)), 0, 15);
    q = clamp(rne(fl32(v / S)) + z, 0, 15): round first, then add z; all
    true fp32 divisions, round half to even.
  * min/max are the raw group extremes (0 is not forced into the range).
  * A constant group (S == 0) stores S = 0, z = 0 and codes 0.
  * Layout: W[N, K] with groups of g consecutive k inside a row; packed byte
    [n, k // 2] holds k even in the low nibble and k odd in the high nibble;
    S fp32 [N, K // g]; z uint8 [N, K // g].
"""
from __future__ import annotations

import numpy as np

QMAX = 15  # 4-bit unsigned code range 0..15


def _as_f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def group_scale_zero(v: np.ndarray):
    """Per-group step S and zero point z for v[..., g] (fp32, min-max, asymmetric).

    Returns (S fp32 [...], z uint8 [...]).
    """
    v = _as_f32(v)
    mn = v.min(axis=-1)
    mx = v.max(axis=-1)
    r = (mx - mn).astype(np.float32)                      # fl32(max - min)
    s = (r / np.float32(QMAX)).astype(np.float32)          # fl32(R / 15), true division
    degenerate = s == 0
    safe = np.where(degenerate, np.float32(1), s).astype(np.float32)
    zf = np.rint((-mn) / safe).astype(np.float32)          # rne(fl32(-min / S))
    z = np.clip(zf, 0, QMAX)
    z = np.where(degenerate, 0, z).astype(np.uint8)
    s = np.where(degenerate, np.float32(0), s).astype(np.float32)
    return s, z


def quantize_codes(w, group: int, chan_scale=None):
    """Codes q [N, K] (uint8 0..15), S [N, K/g] fp32, z [N, K/g] uint8.

    ``w`` is W[N, K] as fp32 values (bf16 weights are widened exactly).
    ``chan_scale`` is the optional per-input-channel AWQ scale s[K] (fp32):
    the group statistics and codes are then those of v = fl32(w * s_k).
    """
    w = _as_f32(w)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    if chan_scale is not None:
        v = (w * _as_f32(chan_scale)[None, :]).astype(np.float32)   # fl32(w * s_k)
    else:
        v = w
    vg = v.reshape(n, k // group, group)
    s, z = group_scale_zero(vg)
    degenerate = (s == 0)[..., None]
    safe = np.where(degenerate, np.float32(1), s[..., None]).astype(np.float32)
    r = np.rint(vg / safe).astype(np.float32)              # rne(fl32(v / S))
    q = np.clip(r + z[..., None].astype(np.float32), 0, QMAX)
    q = np.where(degenerate, 0, q).astype(np.uint8)
    return q.reshape(n, k), s, z


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: even k in the low nibble, odd k in the high nibble."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    if q.shape[-1] % 2:
        raise ValueError("K must be even to pack two codes per byte")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_nibbles``: [.., K/2] bytes -> [.., K] codes."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize_pack(w, group: int, chan_scale=None):
    """(packed [N, K/2] uint8, S [N, K/g] fp32, z [N, K/g] uint8)."""
    q, s, z = quantize_codes(w, group, chan_scale)
    return pack_nibbles(q), s, z


# ---- 8-bit variant ---------------------------------------------------------------
# The same asymmetric min-max formulas with the 8-bit unsigned range 0 .. 255
# ("Quantization：模型量化", xingyuwang.me, section 2: the integer range sets the
# clip; "BNB/GPTQ/AWQ量化全面支持", maplevalley.com.cn: weight-only 8-bit next to
# 4-bit; the mixed 4/8-bit policy keeps key layers at 8 bits, "模型量化指南",
# blog.yoooo.fun, "混合精度（按层 4/8-bit）").  Readings: S = fl32(fl32(max - min)
# / 255), z = clamp(rne(fl32(-min / S)), 0, 255), q = clamp(rne(fl32(v / S)) + z,
# 0, 255); one code byte per weight, codes [N, K] uint8; S fp32 and z uint8
# [N, K / g]; a constant group stores S = 0, z = 0, q = 0.
QMAX8 = 255


def quantize_codes8(w, group: int, chan_scale=None):
    """Codes q [N, K] (uint8 0..255), S [N, K/g] fp32, z [N, K/g] uint8."""
    w = _as_f32(w)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    v = (w * _as_f32(chan_scale)[None, :]).astype(np.float32) if chan_scale is not None else w
    vg = v.reshape(n, k // group, group)
    mn = vg.min(axis=-1)
    mx = vg.max(axis=-1)
    s = ((mx - mn).astype(np.float32) / np.float32(QMAX8)).astype(np.float32)   # fl32(fl32(max-min) / 255)
    degenerate = s == 0
    safe = np.where(degenerate, np.float32(1), s).astype(np.float32)
    z = np.clip(np.rint((-mn) / safe), 0, QMAX8)                             # rne(fl32(-min / S))
    z = np.where(degenerate, 0, z)
    r = np.rint(vg / safe[..., None])                                         # rne(fl32(v / S))
    q = np.clip(r + z[..., None], 0, QMAX8)
    q = np.where(degenerate[..., None], 0, q)
    s = np.where(degenerate, np.float32(0), s).astype(np.float32)
    return q.astype(np.uint8).reshape(n, k), s, z.astype(np.uint8)


def dequantize8(codes, scales, zeros, group: int) -> np.ndarray:
    """W_hat[N, K] = (q - z) * S in fp64 from one code byte per weight."""
    q = np.asarray(codes, dtype=np.float64)
    n, k = q.shape
    s = np.asarray(scales, dtype=np.float64).reshape(n, k // group, 1)
    z = np.asarray(zeros, dtype=np.float64).reshape(n, k // group, 1)
    return ((q.reshape(n, k // group, group) - z) * s).reshape(n, k)


def forward8(x_f32, codes, scales, zeros, group: int) -> np.ndarray:
    """Y[M, N] = X @ W_hat^T for 8-bit codes, fp64."""
    return np.asarray(x_f32, dtype=np.float64) @ dequantize8(codes, scales, zeros, group).T


# ---- symmetric variant --------------------------------------------------------
# "Quantization：模型量化" (xingyuwang.me), section 2, symmetric quantization: a
# symmetric integer range with zero mapped to integer zero, q = round(x / s),
# x_hat = q s (the page's INT8 example uses -127 .. 127), then clipping to the
# integer range.  Readings (listed in the design notes): the 4-bit range is
# -7 .. 7 with s = fl32(max |v| / 7) per group; the code is stored offset by 8
# (1 .. 15) with a zero point of 8 for every group, so (code - z) S = q s and the
# asymmetric decode applies unchanged; an all-zero group stores S = 0, codes 8.
SYM_QMAX = 7
SYM_ZERO = 8


def quantize_codes_sym(w, group: int, chan_scale=None):
    """Stored codes [N, K] (uint8, q + 8 with q in -7..7), S [N, K/g] fp32, z [N, K/g] (all 8)."""
    w = _as_f32(w)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    v = (w * _as_f32(chan_scale)[None, :]).astype(np.float32) if chan_scale is not None else w
    vg = v.reshape(n, k // group, group)
    amax = np.abs(vg).max(axis=-1)                                   # exact
    s = (amax / np.float32(SYM_QMAX)).astype(np.float32)             # fl32(max|v| / 7)
    degenerate = (s == 0)[..., None]
    safe = np.where(degenerate, np.float32(1), s[..., None]).astype(np.float32)
    q = np.clip(np.rint(vg / safe), -SYM_QMAX, SYM_QMAX)               # rne(fl32(v / S)), clipped
    q = np.where(degenerate, 0, q) + SYM_ZERO
    z = np.full(s.shape, SYM_ZERO, dtype=np.uint8)
    return q.astype(np.uint8).reshape(n, k), s, z


def quantize_pack_sym(w, group: int, chan_scale=None):
    """(packed [N, K/2] uint8, S [N, K/g] fp32, z [N, K/g] uint8 = 8) of the symmetric variant."""
    q, s, z = quantize_codes_sym(w, group, chan_scale)
    return pack_nibbles(q), s, z


def dequantize(packed, scales, zeros, group: int) -> np.ndarray:
    """W_hat[N, K] = (q - z) * S in fp64 (exact: a 5-bit integer times an fp32 value)."""
    q = unpack_nibbles(packed).astype(np.float64)
    n, k = q.shape
    s = np.asarray(scales, dtype=np.float64).reshape(n, k // group, 1)
    z = np.asarray(zeros, dtype=np.float64).reshape(n, k // group, 1)
    return ((q.reshape(n, k // group, group) - z) * s).reshape(n, k)


def forward(x_f32, packed, scales, zeros, group: int) -> np.ndarray:
    """Y[M, N] = X[M, K] @ W_hat[N, K]^T, fp64 throughout (the W4A16 linear's exact value)."""
    x = np.asarray(x_f32, dtype=np.float64)
    return x @ dequantize(packed, scales, zeros, group).T


def storage_bytes(n: int, k: int, group: int, bits: int = 4):
    """(code bytes, metadata bytes) of the packed format: bits/8 per weight, fp32 S + u8 z per group."""
    return n * k * bits // 8, (n * k // group) * (4 + 1)
