"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds none of the method's arithmetic: it only draws random
numbers and casts them to the storage types the kernels read (bf16 bit
patterns held in uint16 arrays, fp32, uint8).  Both the CPU oracle and the
HIP path receive the identical bytes it produces.

Workload shapes follow the Qwen2.5-3B-style decoder layer the workloads are
quoted on (hidden 2048, intermediate 11008, 16 query heads / 2 KV heads of
128).  Weights are stored PyTorch-``nn.Linear`` style, W[N, K] with K (the
input features) contiguous.
"""
from __future__ import annotations

import numpy as np

# (name, N = out_features, K = in_features) of one decoder layer.
LAYER_LINEARS = (
    ("q_proj", 2048, 2048),
    ("k_proj", 256, 2048),
    ("v_proj", 256, 2048),
    ("o_proj", 2048, 2048),
    ("gate_proj", 11008, 2048),
    ("up_proj", 11008, 2048),
    ("down_proj", 2048, 11008),
)
LINEAR_SHAPES = {name: (n, k) for name, n, k in LAYER_LINEARS}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round half to even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weight_f32(rng: np.random.Generator, n: int, k: int, std: float = 0.02,
               outlier_frac: float = 0.0, outlier_mul: float = 10.0) -> np.ndarray:
    """fp32 W[n, k] ~ N(0, std) with a seeded fraction of entries multiplied by ``outlier_mul``."""
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    cnt = int(round(outlier_frac * n * k))
    if cnt:
        idx = rng.choice(n * k, cnt, replace=False)
        flat = w.reshape(-1)
        flat[idx] *= np.float32(outlier_mul)
    return w


def activations_f32(rng: np.random.Generator, m: int, k: int, outlier_channels: int,
                    outlier_mul: float = 20.0) -> np.ndarray:
    """fp32 X[m, k] ~ N(0, 1) with ``outlier_channels`` seeded input channels scaled by ``outlier_mul``."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if outlier_channels:
        ch = rng.choice(k, outlier_channels, replace=False)
        x[:, ch] *= np.float32(outlier_mul)
    return x


def single_linear(seed: int = 0):
    """Small single-linear case: W fp32 [256, 256] ~ N(0, 0.02), X bf16 [8, 256] with 4 outlier channels x20."""
    rng = np.random.default_rng(seed)
    w = weight_f32(rng, 256, 256, 0.02)
    x = f32_to_bf16_bits(activations_f32(rng, 8, 256, 4))
    return {"W": w, "X": x, "group": 128}


def layer_weight_bf16(seed: int, name: str) -> np.ndarray:
    """bf16 bits of one linear of the decode/prefill layer: N(0, 0.02) with 0.1 % of entries x10."""
    n, k = LINEAR_SHAPES[name]
    idx = [nm for nm, _, _ in LAYER_LINEARS].index(name)
    rng = np.random.default_rng([seed, idx])
    return f32_to_bf16_bits(weight_f32(rng, n, k, 0.02, outlier_frac=0.001))


def layer_activations_bf16(seed: int, m: int, k: int) -> np.ndarray:
    """bf16 bits of X[m, k] ~ N(0, 1) with 1 % of the input channels scaled x20."""
    rng = np.random.default_rng([seed, 1000 + m, k])
    return f32_to_bf16_bits(activations_f32(rng, m, k, int(round(0.01 * k))))


def calibration_bf16(seed: int = 4, samples: int = 128, tokens: int = 512, k: int = 2048) -> np.ndarray:
    """Calibration activations [samples*tokens, k]: x = z * c_k with z ~ N(0,1), c_k = exp(1.5 N(0,1))."""
    rng = np.random.default_rng(seed)
    c = np.exp(np.float32(1.5) * rng.standard_normal(k, dtype=np.float32)).astype(np.float32)
    z = rng.standard_normal((samples * tokens, k), dtype=np.float32)
    z *= c[None, :]
    return f32_to_bf16_bits(z)


def calibration_rows_bf16(seed: int, rows: int, k: int) -> np.ndarray:
    """A smaller calibration matrix with the same per-channel log-normal magnitudes."""
    rng = np.random.default_rng(seed)
    c = np.exp(np.float32(1.5) * rng.standard_normal(k, dtype=np.float32)).astype(np.float32)
    z = rng.standard_normal((rows, k), dtype=np.float32)
    z *= c[None, :]
    return f32_to_bf16_bits(z)


def fp4_weight_f32(seed: int, n: int, k: int) -> np.ndarray:
    """fp32 W[n, k] ~ N(0, 0.02) for the FP4 (E2M1 + E4M3/16) MLP shapes."""
    rng = np.random.default_rng([seed, n, k])
    return weight_f32(rng, n, k, 0.02)


def random_fp4_operands(seed: int, n: int, k: int):
    """Random but well-formed FP4 operands (E2M1 codes, finite E4M3 block scales, fp32 tensor scale).

    Used where realistic encodings are not needed (throughput runs): codes are
    uniform bytes, block scales are uniform over the finite E4M3 bytes in
    [0x20, 0x5F] (magnitudes 2^-3 .. 2^4, positive), tensor scale 2^-9.
    """
    rng = np.random.default_rng([seed, 77, n, k])
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x60, size=(n, k // 16), dtype=np.uint8)
    return codes, scales, np.float32(2.0 ** -9)
