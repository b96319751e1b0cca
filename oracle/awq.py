"""AWQ grid search over the scale exponent alpha.

Test infrastructure only (see the package docstring).

Sources
  * "Lance-Quant" page (zingnex.cn), section "量化应用：网格搜索与分组策略":
    awq_apply grid-searches the AWQ scale equalisation for each norm and its
    consuming linears, then packs the scaled weights group-wise into INT4;
    section "校准阶段" gives the statistic (per-channel mean |x|) and the
    fallback: with no activation data the method degenerates to plain
    min-max quantization.
  * "Quantization：模型量化" (xingyuwang.me), section 7 "AWQ": activation
    statistics identify salient channels that scaling then protects.
  * The equivalent transform Y = (X * s)(W / s) is exact in real arithmetic,
    OmniQuant tutorial (cyqw.cn), section 2.2.2 (learnable equivalent
    transformation); AWQ uses the same identity with s -> 1/s:
    Y = (X / s)(s W).

The search, as stated by the method: for every alpha on the grid the
candidate scale is s = mean|x|^alpha normalised by sqrt(max(s) * min(s));
W * diag(s) is quantize-dequantized group-wise and scored by the output MSE
of (X / s) Q(W s)^T against X W^T over the calibration tokens; the alpha
with the smallest MSE wins and W * diag(s_best) is packed.

Readings (listed in the design notes): alpha_i = i / n_grid for
i = 0 .. n_grid - 1 (0 included, 1 excluded); the pow, product and square
root are fp64 libm operations and s is rounded once to fp32; a channel with
mean 0 is floored at 1e-8 before the pow; in real arithmetic
(X/s) Q(Ws)^T - X W^T = X E^T with E = Q(Ws)/s - W, which is evaluated in
fp64 (X/s is never rounded); the MSE is the mean of the T x N squared
differences; ties go to the smallest alpha.
"""
from __future__ import annotations

import math

import numpy as np

from . import int4

MEAN_FLOOR = 1e-8


def alpha_grid(n_grid: int):
    return [i / n_grid for i in range(n_grid)]


def candidate_scale(mean_abs, alpha: float) -> np.ndarray:
    """s_k = fl32(t_k / sqrt(max t * min t)), t_k = max(m_k, 1e-8) ** alpha (fp64 libm pow)."""
    m = [max(float(v), MEAN_FLOOR) for v in np.asarray(mean_abs, dtype=np.float32)]
    t = [math.pow(v, alpha) for v in m]
    den = math.sqrt(max(t) * min(t))
    return np.array([v / den for v in t], dtype=np.float64).astype(np.float32)


def error_matrix(w, group: int, s) -> np.ndarray:
    """E = (q - z) S / s_k - W in fp64 for the codes of W * diag(s)."""
    w = np.asarray(w, dtype=np.float32)
    packed, sc, zr = int4.quantize_pack(w, group, s)
    what = int4.dequantize(packed, sc, zr, group)
    return what / np.asarray(s, dtype=np.float64)[None, :] - w.astype(np.float64)


def output_mse(x_f32, e, chunk: int = 2048) -> float:
    """mean over (t, n) of (X E^T)[t, n]^2, fp64 (chunked over n only to bound memory)."""
    x = np.asarray(x_f32, dtype=np.float64)
    total = 0.0
    for n0 in range(0, e.shape[0], chunk):
        d = x @ e[n0:n0 + chunk].T
        total += float(np.sum(d * d))
    return total / (x.shape[0] * e.shape[0])


def search(x_f32, mean_abs, w, group: int, n_grid: int = 20, alphas=None):
    """Exhaustive alpha search.

    Returns dict(best, alphas, mse[n_grid], scale = s_best fp32 [K],
    packed, scales, zeros) where the packed triple is W * diag(s_best).
    ``alphas`` restricts which grid indices are scored (others get +inf);
    by default every index is scored.
    """
    x = np.asarray(x_f32)
    if x.shape[0] == 0:
        raise ValueError("empty calibration data")
    grid = alpha_grid(n_grid)
    idx = range(n_grid) if alphas is None else alphas
    mse = np.full(n_grid, np.inf)
    for i in idx:
        s = candidate_scale(mean_abs, grid[i])
        mse[i] = output_mse(x, error_matrix(w, group, s))
    best = int(np.argmin(mse))            # first minimum: ties go to the smallest alpha
    s_best = candidate_scale(mean_abs, grid[best])
    packed, sc, zr = int4.quantize_pack(w, group, s_best)
    return {"best": best, "alphas": grid, "mse": mse, "scale": s_best,
            "packed": packed, "scales": sc, "zeros": zr}
