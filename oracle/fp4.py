"""FP4 (E2M1) codes with FP8 (E4M3) per-16 block scales and an fp32 tensor scale.

Test infrastructure only (see the package docstring).

Sources
  * "Lance-Quant" page (zingnex.cn), section "量化应用：网格搜索与分组策略":
    the NVFP4 variant packs E2M1 codes with an FP8 E4M3 scale for every
    16-element block (nvfp4_apply --block_size 16), from the same calibration.
  * "Quantization：模型量化" (xingyuwang.me), section 12 "FP8 与 FP4":
    E4M3 = 1 sign + 4 exponent + 3 mantissa bits, E5M2 = 1 + 5 + 2.

Readings (the pages give only the names and bit splits):
  * E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0;
    exponent 0 is subnormal (0.5 * m).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
  * E4M3: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0;
    exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN;
    no infinities; largest finite value 448.
  * Layout: codes [N, K/2] uint8 with even k in the low nibble; block scales
    [N, K/16] uint8 (one E4M3 byte for k in [16 j, 16 j + 16)); ts fp32.
  * W_hat[n, k] = e2m1(code) * e4m3(block scale) * ts.
  * Encoder (parity unpinned beyond its round-trip bound): ts = fl32(amax(|W|)
    / 2688); block byte = E4M3 round-to-nearest-even, saturating, of
    fl32(amax_block / fl32(6 ts)) (0 for an all-zero block); code = nearest
    E2M1 magnitude of fl32(|w| / fl32(e4m3(b) ts)), ties to the even code,
    saturating at 6, with the sign bit set for negative non-zero magnitudes.
"""
from __future__ import annotations

import numpy as np

from .int4 import pack_nibbles, unpack_nibbles

BLOCK = 16


def e2m1_value(code) -> np.ndarray:
    """fp64 value of 4-bit E2M1 codes, from the bit fields."""
    c = np.asarray(code).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1)))
    return sign * mag


def e4m3_value(byte) -> np.ndarray:
    """fp64 value of E4M3 bytes (OCP 'FN' variant), from the bit fields."""
    b = np.asarray(byte).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _nearest_code(a: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of the ascending ``values`` (ties -> even index), saturating."""
    a = np.minimum(a, values[-1])
    hi = np.clip(np.searchsorted(values, a, side="left"), 1, len(values) - 1)
    lo = hi - 1
    dlo = a - values[lo]
    dhi = values[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


_E4M3_POS = e4m3_value(np.arange(0x7F))           # finite non-negative codes 0x00..0x7E, ascending
_E2M1_POS = e2m1_value(np.arange(8))              # 0, .5, 1, 1.5, 2, 3, 4, 6


def e4m3_encode(a) -> np.ndarray:
    """Round non-negative values to E4M3 bytes (nearest, ties to even, saturate at 448)."""
    return _nearest_code(np.asarray(a, dtype=np.float64), _E4M3_POS).astype(np.uint8)


def encode(w):
    """(codes [N, K/2] uint8, block scales [N, K/16] uint8, ts fp32) for W[N, K] fp32."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    ts = np.float32(amax / np.float32(6 * 448))
    if ts == 0:
        ts = np.float32(1)
    wb = w.reshape(n, k // BLOCK, BLOCK)
    amax_b = np.max(np.abs(wb), axis=-1)
    target = (amax_b / np.float32(np.float32(6) * ts)).astype(np.float32)
    b = e4m3_encode(target)
    scale_b = (e4m3_value(b).astype(np.float32) * ts).astype(np.float32)
    safe = np.where(scale_b == 0, np.float32(1), scale_b).astype(np.float32)
    r = (np.abs(wb) / safe[..., None]).astype(np.float32)
    mag = _nearest_code(r.astype(np.float64), _E2M1_POS)
    mag = np.where((scale_b == 0)[..., None], 0, mag)
    code = np.where((wb < 0) & (mag != 0), mag | 8, mag).astype(np.uint8)
    return pack_nibbles(code.reshape(n, k)), b, ts


def dequantize(codes, block_scales, ts) -> np.ndarray:
    """W_hat[N, K] = e2m1 * e4m3 * ts in fp64."""
    c = unpack_nibbles(codes)
    n, k = c.shape
    sc = np.repeat(e4m3_value(block_scales), BLOCK, axis=-1).reshape(n, k)
    return e2m1_value(c) * sc * float(ts)


def forward(x_f32, codes, block_scales, ts) -> np.ndarray:
    """Y[M, N] = X @ W_hat^T, fp64."""
    return np.asarray(x_f32, dtype=np.float64) @ dequantize(codes, block_scales, ts).T
