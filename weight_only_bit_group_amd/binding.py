"""Thin torch binding of libaq: the C entry points under the same names.

Argument marshalling only -- every step of the computation runs in the
library's HIP kernels.  Tensors must be CUDA (HIP) tensors; outputs are
allocated with torch when not supplied; calls are enqueued on the current
torch stream of the tensors' device.  Status 1 raises ValueError, status 2
RuntimeError, with the library's message.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from ._lib import AQ_BF16, AQ_F32, check


def _stream(t: torch.Tensor) -> int:
    # raw handle of torch's current stream on the tensor's device (cheap accessor)
    return torch._C._cuda_getCurrentRawStream(t.device.index)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _wdtype(w: torch.Tensor) -> int:
    if w.dtype == torch.float32:
        return AQ_F32
    if w.dtype == torch.bfloat16:
        return AQ_BF16
    raise ValueError(f"W must be float32 or bfloat16 (got {w.dtype})")


def _packed_outputs(w_like: torch.Tensor, n: int, k: int, group: int, packed, scales, zeros):
    dev = w_like.device
    if packed is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((n, k // group), dtype=torch.float32, device=dev)
    if zeros is None:
        zeros = torch.empty((n, k // group), dtype=torch.uint8, device=dev)
    return packed, scales, zeros


def aq_quantize_pack(W: torch.Tensor, group: int, chan_scale: torch.Tensor | None = None, *,
                     packed=None, scales=None, zeros=None, sym: bool = False):
    """(packed [N, K/2] u8, scales [N, K/g] f32, zeros [N, K/g] u8) of W[N, K] (f32 or bf16).

    sym=True calls aq_quantize_pack_sym (symmetric codes, zero point 8).
    """
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    _need(W, "W", W.dtype)
    n, k = W.shape
    if k % group:
        raise ValueError("K must be a multiple of group")
    if chan_scale is not None:
        _need(chan_scale, "chan_scale", torch.float32, 1)
    packed, scales, zeros = _packed_outputs(W, n, k, group, packed, scales, zeros)
    fn = "aq_quantize_pack_sym" if sym else "aq_quantize_pack"
    st = getattr(_lib.load(), fn)(W.data_ptr(), _wdtype(W), n, k, group, _ptr(chan_scale), packed.data_ptr(),
                                  scales.data_ptr(), zeros.data_ptr(), _stream(W))
    check(st, fn)
    return packed, scales, zeros


def _workspace(ws, need: int, device):
    """(pointer, bytes) of a workspace: allocated here when `ws` is None and `need` > 0."""
    if ws is None:
        if need <= 0:
            return None, 0
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if ws.numel() == 0:
        return None, 0
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ws, ws.numel() * ws.element_size()


def _product(fn_name, X, packed, scales, zeros, group, out, workspace=None):
    _need(X, "X", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 2)
    _need(scales, "scales", torch.float32, 2)
    _need(zeros, "zeros", torch.uint8, 2)
    m, k = X.shape
    n = packed.shape[0]
    if packed.shape[1] * 2 != k:
        raise ValueError("packed must be [N, K/2] for X [M, K]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=X.device)
    _need(out, "Y", torch.float32, 2)
    lib = _lib.load()
    if fn_name == "aq_w4a16_gemm":
        ws, nbytes = _workspace(workspace, int(lib.aq_w4a16_gemm_workspace(m, n, k, group)), X.device)
        st = lib.aq_w4a16_gemm(X.data_ptr(), m, k, packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), n, group,
                               out.data_ptr(), _ptr(ws), nbytes, _stream(X))
    else:
        st = getattr(lib, fn_name)(X.data_ptr(), m, k, packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                   n, group, out.data_ptr(), _stream(X))
    check(st, fn_name)
    return out


def aq_w4a16_gemv(X, packed, scales, zeros, group: int, out=None):
    """Y[M, N] fp32 = X[M, K] (bf16, 1 <= M <= 16) times the dequantized packed weight, transposed."""
    return _product("aq_w4a16_gemv", X, packed, scales, zeros, group, out)


def aq_w4a16_gemm_workspace(M: int, N: int, K: int, group: int) -> int:
    return int(_lib.load().aq_w4a16_gemm_workspace(M, N, K, group))


def aq_w4a16_gemm(X, packed, scales, zeros, group: int, out=None, workspace=None):
    """Y[M, N] fp32 = X[M, K] (bf16, any M) times the dequantized packed weight, transposed (MFMA).

    workspace: None allocates the staging matrix when the size takes the staged path;
    a uint8 device tensor is used as given (an empty one selects the fused path).
    """
    return _product("aq_w4a16_gemm", X, packed, scales, zeros, group, out, workspace)


def aq_act_absmean_workspace(T: int, K: int) -> int:
    return int(_lib.load().aq_act_absmean_workspace(T, K))


def aq_act_absmean(X, sum_abs, total_count: int, mean_out=None, workspace=None):
    """sum_abs[K] (fp64) += sum_t |X[t, K]|; mean_out[K] = fl32(sum_abs / total_count) if given."""
    _need(X, "X", torch.bfloat16, 2)
    _need(sum_abs, "sum_abs", torch.float64, 1)
    t, k = X.shape
    if mean_out is not None:
        _need(mean_out, "mean_out", torch.float32, 1)
    need = aq_act_absmean_workspace(t, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=X.device)
    st = _lib.load().aq_act_absmean(X.data_ptr(), t, k, sum_abs.data_ptr(), _ptr(mean_out), total_count,
                                    workspace.data_ptr(), workspace.numel(), _stream(X))
    check(st, "aq_act_absmean")
    return sum_abs, mean_out


def aq_act_absmean_noalloc(X, sum_abs, total_count: int, mean_out=None):
    """aq_act_absmean with the library's own scratch (no workspace, nothing allocated)."""
    _need(X, "X", torch.bfloat16, 2)
    _need(sum_abs, "sum_abs", torch.float64, 1)
    t, k = X.shape
    if mean_out is not None:
        _need(mean_out, "mean_out", torch.float32, 1)
    st = _lib.load().aq_act_absmean_noalloc(X.data_ptr(), t, k, sum_abs.data_ptr(), _ptr(mean_out), total_count,
                                            _stream(X))
    check(st, "aq_act_absmean_noalloc")
    return sum_abs, mean_out


def aq_awq_search_workspace(T: int, N: int, K: int, group: int, n_grid: int = 20) -> int:
    return int(_lib.load().aq_awq_search_workspace(T, N, K, group, n_grid))


def aq_awq_search(X_sub, absmean_host, W, group: int, n_grid: int = 20, workspace=None):
    """Alpha-grid AWQ search.  ``absmean_host`` is a host fp32 array/tensor [K].

    Returns dict(mse [n_grid] f64, best [1] i32, best_scale [K] f32, packed, scales, zeros) on the device.
    """
    _need(X_sub, "X_sub", torch.bfloat16, 2)
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    _need(W, "W", W.dtype)
    t, k = X_sub.shape
    n = W.shape[0]
    if W.shape[1] != k:
        raise ValueError("W must be [N, K] for X_sub [T, K]")
    m = np.ascontiguousarray(absmean_host.cpu().numpy() if isinstance(absmean_host, torch.Tensor) else absmean_host,
                             dtype=np.float32)
    if m.shape != (k,):
        raise ValueError("absmean_host must have K entries")
    dev = X_sub.device
    mse = torch.empty(n_grid, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    best_scale = torch.empty(k, dtype=torch.float32, device=dev)
    packed, scales, zeros = _packed_outputs(W, n, k, group, None, None, None)
    need = aq_awq_search_workspace(t, n, k, group, n_grid)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = _lib.load().aq_awq_search(X_sub.data_ptr(), t, m.ctypes.data, W.data_ptr(), _wdtype(W), n, k, group, n_grid,
                                   mse.data_ptr(), best.data_ptr(), best_scale.data_ptr(), packed.data_ptr(),
                                   scales.data_ptr(), zeros.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream(X_sub))
    check(st, "aq_awq_search")
    return {"mse": mse, "best": best, "best_scale": best_scale, "packed": packed, "scales": scales, "zeros": zeros}


def aq_awq_fold_norm(norm_w, chan_scale, out=None):
    """folded [K] fp32 = fl32(norm_w / chan_scale) on the device (norm_w fp32 or bf16; other float
    dtypes are widened to fp32 first, exactly)."""
    if norm_w.dtype not in (torch.float32, torch.bfloat16):
        norm_w = norm_w.float()
    _need(norm_w, "norm_w", norm_w.dtype, 1)
    _need(chan_scale, "chan_scale", torch.float32, 1)
    k = norm_w.shape[0]
    if chan_scale.shape[0] != k:
        raise ValueError("norm_w and chan_scale must have the same length")
    if out is None:
        out = torch.empty(k, dtype=torch.float32, device=norm_w.device)
    _need(out, "folded", torch.float32, 1)
    st = _lib.load().aq_awq_fold_norm(norm_w.data_ptr(), _wdtype(norm_w), chan_scale.data_ptr(), k, out.data_ptr(),
                                      _stream(norm_w))
    check(st, "aq_awq_fold_norm")
    return out


def aq_fp4_gemm_workspace(M: int, N: int, K: int) -> int:
    return int(_lib.load().aq_fp4_gemm_workspace(M, N, K))


def aq_fp4_gemm(X, codes, block_scales, tensor_scale: float, out=None, workspace=None):
    """Y[M, N] fp32 = tensor_scale * X[M, K] times (e2m1 * e4m3)^T for codes [N, K/2], block_scales [N, K/16]."""
    _need(X, "X", torch.bfloat16, 2)
    _need(codes, "codes", torch.uint8, 2)
    _need(block_scales, "block_scales", torch.uint8, 2)
    m, k = X.shape
    n = codes.shape[0]
    if codes.shape[1] * 2 != k or block_scales.shape != (n, k // 16):
        raise ValueError("codes must be [N, K/2] and block_scales [N, K/16]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=X.device)
    _need(out, "Y", torch.float32, 2)
    lib = _lib.load()
    ws, nbytes = _workspace(workspace, int(lib.aq_fp4_gemm_workspace(m, n, k)), X.device)
    st = lib.aq_fp4_gemm(X.data_ptr(), m, k, codes.data_ptr(), block_scales.data_ptr(), float(tensor_scale),
                         n, out.data_ptr(), _ptr(ws), nbytes, _stream(X))
    check(st, "aq_fp4_gemm")
    return out


def aq_fp4_quantize_workspace(N: int, K: int) -> int:
    return int(_lib.load().aq_fp4_quantize_workspace(N, K))


def aq_fp4_quantize(W, *, codes=None, block_scales=None, tensor_scale=None, workspace=None):
    """(codes [N, K/2] u8, block_scales [N, K/16] u8, tensor_scale [1] f32) of W[N, K] (f32 or bf16), on the device."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    _need(W, "W", W.dtype)
    n, k = W.shape
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    dev = W.device
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    if block_scales is None:
        block_scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
    if tensor_scale is None:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=dev)
    need = aq_fp4_quantize_workspace(n, k)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    st = _lib.load().aq_fp4_quantize(W.data_ptr(), _wdtype(W), n, k, codes.data_ptr(), block_scales.data_ptr(),
                                     tensor_scale.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(W))
    check(st, "aq_fp4_quantize")
    return codes, block_scales, tensor_scale


def aq_quantize_pack8(W: torch.Tensor, group: int, chan_scale: torch.Tensor | None = None, *,
                      codes=None, scales=None, zeros=None):
    """(codes [N, K] u8, scales [N, K/g] f32, zeros [N, K/g] u8) of W[N, K] (f32 or bf16), 8-bit codes."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N, K]")
    _need(W, "W", W.dtype)
    n, k = W.shape
    if k % group:
        raise ValueError("K must be a multiple of group")
    if chan_scale is not None:
        _need(chan_scale, "chan_scale", torch.float32, 1)
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.uint8, device=W.device)
    _, scales, zeros = _packed_outputs(W, n, k, group, codes, scales, zeros)
    st = _lib.load().aq_quantize_pack8(W.data_ptr(), _wdtype(W), n, k, group, _ptr(chan_scale), codes.data_ptr(),
                                       scales.data_ptr(), zeros.data_ptr(), _stream(W))
    check(st, "aq_quantize_pack8")
    return codes, scales, zeros


def aq_w8a16_gemm_workspace(M: int, N: int, K: int, group: int) -> int:
    return int(_lib.load().aq_w8a16_gemm_workspace(M, N, K, group))


def _product8(fn_name, X, codes, scales, zeros, group, out, workspace=None):
    _need(X, "X", torch.bfloat16, 2)
    _need(codes, "codes", torch.uint8, 2)
    _need(scales, "scales", torch.float32, 2)
    _need(zeros, "zeros", torch.uint8, 2)
    m, k = X.shape
    n = codes.shape[0]
    if codes.shape[1] != k:
        raise ValueError("codes must be [N, K] for X [M, K]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=X.device)
    _need(out, "Y", torch.float32, 2)
    lib = _lib.load()
    if fn_name == "aq_w8a16_gemm":
        need = int(lib.aq_w8a16_gemm_workspace(m, n, k, group))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=X.device)
        st = lib.aq_w8a16_gemm(X.data_ptr(), m, k, codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), n, group,
                               out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(X))
    else:
        st = lib.aq_w8a16_gemv(X.data_ptr(), m, k, codes.data_ptr(), scales.data_ptr(), zeros.data_ptr(), n, group,
                               out.data_ptr(), _stream(X))
    check(st, fn_name)
    return out


def aq_w8a16_gemv(X, codes, scales, zeros, group: int, out=None):
    """Y[M, N] fp32 = X[M, K] (bf16, 1 <= M <= 16) times the dequantized 8-bit weight, transposed."""
    return _product8("aq_w8a16_gemv", X, codes, scales, zeros, group, out)


def aq_w8a16_gemm(X, codes, scales, zeros, group: int, out=None, workspace=None):
    """Y[M, N] fp32 = X[M, K] (bf16, any M) times the dequantized 8-bit weight (staged bf16 + MFMA)."""
    return _product8("aq_w8a16_gemm", X, codes, scales, zeros, group, out, workspace)
