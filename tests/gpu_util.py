"""Helpers for the GPU parity tests: device transfer and the tolerance rule."""
import sys

import numpy as np
import torch


def step(msg: str) -> None:
    """Name the case before a GPU step (so a fault can be attributed)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


# Output tolerance (W4A16 / FP4 products against the fp64 dequantized reference):
# normwise max relative error <= 2e-2 and mean absolute error <= 1e-3.
MAX_REL = 2e-2
MEAN_ABS = 1e-3


def check_close(y: np.ndarray, ref: np.ndarray, what: str):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite outputs"
    err = np.abs(y - ref)
    scale = max(np.abs(ref).max(), 1e-30)
    max_rel = err.max() / scale
    mean_abs = err.mean()
    floor = 1e-2 * np.sqrt(np.mean(ref * ref)) + 1e-30
    elem_rel = (err / np.maximum(np.abs(ref), floor)).max()
    print(f"[gpu] {what}: max_rel={max_rel:.3e} mean_abs={mean_abs:.3e} elementwise_rel(floor)={elem_rel:.3e}",
          flush=True)
    assert max_rel <= MAX_REL, f"{what}: max relative error {max_rel:.3e}"
    assert mean_abs <= MEAN_ABS, f"{what}: mean absolute error {mean_abs:.3e}"
    return max_rel, mean_abs
