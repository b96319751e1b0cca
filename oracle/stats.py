"""Per-input-channel mean |x| (the AWQ activation statistic).

Test infrastructure only (see the package docstring).

Source: "Lance-Quant" page (zingnex.cn), section "校准阶段：任务感知的数据收集":
the calibration hooks on every target linear keep, per input channel, the
average absolute activation magnitude; statistics of several runs are then
merged.  AWQ's use of average channel activation magnitudes: "BNB/GPTQ/AWQ量化
全面支持" (maplevalley.com.cn), the AWQ paragraph.

Reading: the mean is over all T tokens seen; the sum of |x| is formed
exactly (``math.fsum`` is correctly rounded), rounded once to fp64, divided by
the token count in fp64 and rounded to fp32.
"""
from __future__ import annotations

import math

import numpy as np


def abs_sum(x_f32) -> np.ndarray:
    """fp64 correctly rounded sum of |x[t, k]| over t, for every channel k."""
    x = np.abs(np.asarray(x_f32, dtype=np.float64))
    return np.array([math.fsum(x[:, k].tolist()) for k in range(x.shape[1])], dtype=np.float64)


def mean_from_sum(sum_abs, count: int) -> np.ndarray:
    """m_k = fl32(sum_k / count), the division in fp64."""
    return (np.asarray(sum_abs, dtype=np.float64) / float(count)).astype(np.float32)


def absmean(x_f32) -> np.ndarray:
    """m[k] = fl32(fl64(sum_t |x[t, k]|) / T)."""
    x = np.asarray(x_f32)
    if x.shape[0] == 0:
        raise ValueError("empty calibration data")
    return mean_from_sum(abs_sum(x), x.shape[0])
