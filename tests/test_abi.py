"""Host-side checks of the C ABI (no GPU needed).

The library loads, exports every entry point the header declares, rejects
invalid arguments with AQ_EINVAL before touching the GPU, and reports the
injected runtime failure with AQ_ERUNTIME.  None of these calls launches a
kernel: validation precedes every launch, and the fault switch returns before
any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from weight_only_bit_group_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aq.h")

FAKE = 0x10000          # 64 KiB-aligned fake device address (never dereferenced)
FAKE_ODD = 0x10002      # misaligned fake address


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("aq_quantize_pack", "aq_w4a16_gemv", "aq_w4a16_gemm", "aq_act_absmean", "aq_awq_search",
              "aq_fp4_gemm", "aq_fp4_quantize", "aq_last_error"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES), "binding prototypes must mirror the header"


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    for name in _declared():
        assert re.search(rf"\bT {name}\b", out), name


def _qp(lib, fn="aq_quantize_pack", **kw):
    a = dict(W=FAKE, dt=1, N=16, K=128, g=64, s=None, p=FAKE, sc=FAKE, z=FAKE)
    a.update(kw)
    return getattr(lib, fn)(a["W"], a["dt"], a["N"], a["K"], a["g"], a["s"], a["p"], a["sc"], a["z"], None)


@pytest.mark.parametrize("kw,frag", [
    (dict(g=48), "group"), (dict(g=256), "group"), (dict(K=96), "multiple"), (dict(K=0), "K"),
    (dict(N=-1), "N"), (dict(dt=7), "dtype"), (dict(W=None), "W"), (dict(W=FAKE_ODD), "aligned"),
    (dict(p=None), "packed"), (dict(s=FAKE_ODD), "chan_scale"), (dict(K=1 << 31), "K"),
])
def test_quantize_pack_einval(lib, kw, frag):
    for fn in ("aq_quantize_pack", "aq_quantize_pack_sym", "aq_quantize_pack8"):
        assert _qp(lib, fn, **kw) == _lib.AQ_EINVAL
        assert frag in _lib.last_error()


def _prod(lib, fn, **kw):
    a = dict(X=FAKE, M=1, K=256, P=FAKE, S=FAKE, Z=FAKE, N=64, g=64, Y=FAKE, ws=None, wsb=0)
    a.update(kw)
    args = [a["X"], a["M"], a["K"], a["P"], a["S"], a["Z"], a["N"], a["g"], a["Y"]]
    if fn == "aq_w4a16_gemm":
        args += [a["ws"], a["wsb"]]
    return getattr(lib, fn)(*args, None)


def _prod8(lib, fn, **kw):
    a = dict(X=FAKE, M=1, K=256, C=FAKE, S=FAKE, Z=FAKE, N=64, g=64, Y=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    args = [a["X"], a["M"], a["K"], a["C"], a["S"], a["Z"], a["N"], a["g"], a["Y"]]
    if fn == "aq_w8a16_gemm":
        args += [a["ws"], a["wsb"]]
    return getattr(lib, fn)(*args, None)


def test_int8_products_einval(lib):
    assert lib.aq_w8a16_gemm_workspace(4096, 64, 256, 64) == 64 * 256 * 2
    assert lib.aq_w8a16_gemm_workspace(4096, 64, 250, 64) == 0
    for kw in (dict(M=0), dict(M=17), dict(g=16), dict(K=100), dict(X=None), dict(C=FAKE + 8), dict(Y=FAKE + 2)):
        assert _prod8(lib, "aq_w8a16_gemv", **kw) == _lib.AQ_EINVAL, kw
    for kw in (dict(M=-1), dict(g=16), dict(ws=None), dict(ws=FAKE + 16), dict(wsb=64 * 256 * 2 - 1),
               dict(K=1 << 22), dict(N=1 << 22)):
        assert _prod8(lib, "aq_w8a16_gemm", **kw) == _lib.AQ_EINVAL, kw


def _fp4(lib, X=FAKE, M=1, K=64, C=FAKE, B=FAKE, ts=1.0, N=8, Y=FAKE, ws=None, wsb=0):
    return lib.aq_fp4_gemm(X, M, K, C, B, ts, N, Y, ws, wsb, None)


@pytest.mark.parametrize("kw", [dict(M=0), dict(M=17), dict(g=16), dict(K=100), dict(X=None), dict(X=FAKE_ODD),
                                dict(P=FAKE + 8), dict(Y=None), dict(N=-3), dict(Y=FAKE + 2)])
def test_gemv_einval(lib, kw):
    assert _prod(lib, "aq_w4a16_gemv", **kw) == _lib.AQ_EINVAL


@pytest.mark.parametrize("kw", [dict(M=-1), dict(g=16), dict(K=100), dict(S=None), dict(Z=None), dict(K=0),
                                dict(K=1 << 22), dict(N=1 << 22)])
def test_gemm_einval(lib, kw):
    assert _prod(lib, "aq_w4a16_gemm", **kw) == _lib.AQ_EINVAL


def test_gemm_workspace_selects_the_staged_path(lib, monkeypatch):
    """The staging matrix is N * K bf16 for large M, 0 below the threshold or for invalid
    arguments; a large enough but misaligned workspace is rejected, a short one means
    the fused path (no error)."""
    need = lib.aq_w4a16_gemm_workspace(4096, 11008, 2048, 64)
    assert need == 11008 * 2048 * 2
    # few output tiles: K slices, their fp32 partials (86 tiles at M = 64: 3 slices of 704 k)
    assert lib.aq_w4a16_gemm_workspace(64, 11008, 2048, 64) == 3 * 64 * 11008 * 4
    # 512 x 2048 (32 tiles): 6 slices of 384 k (the last 128); with staging at M = 4096
    # (32 tiles of N = 256) the partials follow the staging matrix
    assert lib.aq_w4a16_gemm_workspace(512, 2048, 2048, 64) == 6 * 512 * 2048 * 4
    assert lib.aq_w4a16_gemm_workspace(4096, 256, 2048, 64) == 256 * 2048 * 2 + 6 * 4096 * 256 * 4
    # 4 tiles: the most slices (8)
    assert lib.aq_w4a16_gemm_workspace(512, 256, 2048, 64) == 8 * 512 * 256 * 4
    # too short to split (fewer than two slices of four stages), or many tiles: nothing
    assert lib.aq_w4a16_gemm_workspace(512, 2048, 448, 64) == 0
    assert lib.aq_w4a16_gemm_workspace(2047, 11008, 2048, 64) == 0
    assert lib.aq_w4a16_gemm_workspace(4096, 11008, 2048, 48) == 0
    assert lib.aq_w4a16_gemm_workspace(4096, 11008, 2000, 64) == 0
    assert lib.aq_fp4_gemm_workspace(2048, 14336, 4096) == 14336 * 4096 * 2
    assert lib.aq_fp4_gemm_workspace(16, 14336, 4096) == 0
    kw = dict(M=4096, N=512, K=256)
    need = lib.aq_w4a16_gemm_workspace(4096, 512, 256, 64)
    assert _prod(lib, "aq_w4a16_gemm", ws=FAKE + 16, wsb=need, **kw) == _lib.AQ_EINVAL
    assert "workspace" in _lib.last_error()
    assert _fp4(lib, M=4096, K=256, N=512, ws=FAKE + 16, wsb=need) == _lib.AQ_EINVAL
    monkeypatch.setenv("AQ_FAULT_INJECT", "launch")
    assert _prod(lib, "aq_w4a16_gemm", ws=FAKE + 16, wsb=need - 1, **kw) == _lib.AQ_ERUNTIME   # fused path
    assert _prod(lib, "aq_w4a16_gemm", ws=FAKE, wsb=need, **kw) == _lib.AQ_ERUNTIME


def test_empty_products_are_noops(lib):
    assert _prod(lib, "aq_w4a16_gemm", M=0) == _lib.AQ_OK
    assert _prod(lib, "aq_w4a16_gemm", N=0) == _lib.AQ_OK
    assert _prod(lib, "aq_w4a16_gemv", N=0) == _lib.AQ_OK
    assert _qp(lib, N=0) == _lib.AQ_OK
    assert _fp4(lib, M=0) == _lib.AQ_OK


def test_absmean_einval(lib):
    ws = lib.aq_act_absmean_workspace(1024, 256)
    assert ws > 0
    f = lib.aq_act_absmean
    assert f(FAKE, 0, 256, FAKE, None, 0, FAKE, ws, None) == _lib.AQ_EINVAL        # empty calibration data
    assert "empty calibration" in _lib.last_error()
    assert f(FAKE, 1024, 250, FAKE, None, 1024, FAKE, ws, None) == _lib.AQ_EINVAL   # K % 8
    assert f(FAKE, 1024, 256, FAKE, None, 100, FAKE, ws, None) == _lib.AQ_EINVAL    # count < T
    assert f(FAKE, 1024, 256, FAKE, None, 1024, FAKE, ws - 8, None) == _lib.AQ_EINVAL
    assert f(FAKE, 1024, 256, FAKE + 4, None, 1024, FAKE, ws, None) == _lib.AQ_EINVAL
    assert f(FAKE, 1024, 256, FAKE, FAKE + 1, 1024, FAKE, ws, None) == _lib.AQ_EINVAL


def test_absmean_noalloc_einval(lib):
    """The allocation-free abs-mean: the same argument checks as aq_act_absmean, and sizes whose
    partial sums exceed its 8 MiB scratch are refused before anything runs (every K up to 2^20
    fits)."""
    f = lib.aq_act_absmean_noalloc
    assert f(FAKE, 0, 256, FAKE, None, 0, None) == _lib.AQ_EINVAL
    assert "empty calibration" in _lib.last_error()
    assert f(FAKE, 1024, 250, FAKE, None, 1024, None) == _lib.AQ_EINVAL     # K % 8
    assert f(FAKE, 1024, 256, FAKE, None, 100, None) == _lib.AQ_EINVAL     # count < T
    assert f(FAKE, 1024, 256, FAKE + 4, None, 1024, None) == _lib.AQ_EINVAL
    assert f(None, 1024, 256, FAKE, None, 1024, None) == _lib.AQ_EINVAL
    big = 1048584                                                          # partials of 8.4 MB
    assert lib.aq_act_absmean_workspace(1 << 20, big) > 8 << 20
    assert f(FAKE, 1 << 20, big, FAKE, None, 1 << 20, None) == _lib.AQ_EINVAL
    assert "scratch" in _lib.last_error()
    assert lib.aq_act_absmean_workspace(1 << 20, 1 << 20) <= 8 << 20


def test_search_einval(lib):
    T, N, K, g, ng = 64, 32, 128, 64, 20
    ws = lib.aq_awq_search_workspace(T, N, K, g, ng)
    assert ws > 0
    m = np.ones(K, np.float32)
    mp = m.ctypes.data

    def call(**kw):
        a = dict(X=FAKE, T=T, m=mp, W=FAKE, dt=1, N=N, K=K, g=g, ng=ng, mse=FAKE, best=FAKE, bs=FAKE,
                 p=FAKE, sc=FAKE, z=FAKE, ws=FAKE, wsb=ws)
        a.update(kw)
        return lib.aq_awq_search(a["X"], a["T"], a["m"], a["W"], a["dt"], a["N"], a["K"], a["g"], a["ng"], a["mse"],
                                 a["best"], a["bs"], a["p"], a["sc"], a["z"], a["ws"], a["wsb"], None)

    assert call(T=0) == _lib.AQ_EINVAL and "empty calibration" in _lib.last_error()
    assert call(ng=0) == _lib.AQ_EINVAL
    assert call(ng=65) == _lib.AQ_EINVAL
    assert call(K=96) == _lib.AQ_EINVAL
    assert call(wsb=ws - 1) == _lib.AQ_EINVAL and "workspace" in _lib.last_error()
    assert call(m=None) == _lib.AQ_EINVAL
    assert call(ws=FAKE + 16) == _lib.AQ_EINVAL
    bad = m.copy()
    bad[5] = np.nan
    assert call(m=bad.ctypes.data) == _lib.AQ_EINVAL
    bad[5] = -1
    assert call(m=bad.ctypes.data) == _lib.AQ_EINVAL
    assert lib.aq_awq_search_workspace(0, N, K, g, ng) == 0
    # the error GEMM's 32-bit offsets: T, N and K below 2^22 (refused before any launch)
    for kw in (dict(T=1 << 22), dict(N=1 << 22), dict(K=1 << 22)):
        assert call(**kw) == _lib.AQ_EINVAL and "2^22" in _lib.last_error(), kw
    assert lib.aq_awq_search_workspace(1 << 22, N, K, g, ng) == 0
    assert lib.aq_awq_search_workspace(T, 1 << 22, K, g, ng) == 0
    assert lib.aq_awq_search_workspace(T, N, 1 << 22, g, ng) == 0
    assert lib.aq_awq_search_workspace(T, N, (1 << 22) - 64, g, ng) > 0


def test_fold_norm_einval(lib):
    f = lib.aq_awq_fold_norm
    assert f(FAKE, 0, FAKE, 0, FAKE, None) == _lib.AQ_EINVAL
    assert f(FAKE, 0, FAKE, 1 << 30, FAKE, None) == _lib.AQ_EINVAL
    assert f(FAKE, 5, FAKE, 64, FAKE, None) == _lib.AQ_EINVAL and "w_dtype" in _lib.last_error()
    assert f(None, 0, FAKE, 64, FAKE, None) == _lib.AQ_EINVAL
    assert f(FAKE + 2, 0, FAKE, 64, FAKE, None) == _lib.AQ_EINVAL   # fp32 norm weight: 4-byte aligned
    assert f(FAKE, 0, FAKE + 1, 64, FAKE, None) == _lib.AQ_EINVAL
    assert f(FAKE, 0, FAKE, 64, None, None) == _lib.AQ_EINVAL


def test_fp4_einval(lib):
    assert _fp4(lib, K=48) == _lib.AQ_EINVAL     # K % 32
    assert _fp4(lib, ts=float("inf")) == _lib.AQ_EINVAL
    assert _fp4(lib, ts=float("nan")) == _lib.AQ_EINVAL
    assert _fp4(lib, M=-1) == _lib.AQ_EINVAL
    assert _fp4(lib, C=FAKE_ODD) == _lib.AQ_EINVAL
    assert _fp4(lib, M=17, K=1 << 22) == _lib.AQ_EINVAL
    assert _fp4(lib, M=17, N=1 << 22) == _lib.AQ_EINVAL


def _fp4q(lib, W=FAKE, dt=0, N=8, K=64, C=FAKE, B=FAKE, T=FAKE, ws=FAKE, wsb=None):
    wsb = lib.aq_fp4_quantize_workspace(N, K) if wsb is None else wsb
    return lib.aq_fp4_quantize(W, dt, N, K, C, B, T, ws, wsb, None)


def test_fp4_quantize_einval(lib):
    assert lib.aq_fp4_quantize_workspace(8, 64) >= 4
    assert lib.aq_fp4_quantize_workspace(8, 24) == 0
    assert _fp4q(lib, K=24) == _lib.AQ_EINVAL        # K % 16
    assert _fp4q(lib, K=0) == _lib.AQ_EINVAL
    assert _fp4q(lib, dt=7) == _lib.AQ_EINVAL
    assert _fp4q(lib, N=-1) == _lib.AQ_EINVAL
    assert _fp4q(lib, W=FAKE + 8) == _lib.AQ_EINVAL  # W must be 16-byte aligned
    assert _fp4q(lib, C=FAKE + 4) == _lib.AQ_EINVAL  # codes 8-byte aligned
    assert _fp4q(lib, T=None) == _lib.AQ_EINVAL
    assert _fp4q(lib, wsb=0) == _lib.AQ_EINVAL       # workspace too small
    assert "workspace" in _lib.last_error()


def test_injected_runtime_failure(lib, monkeypatch):
    """AQ_FAULT_INJECT=launch: valid arguments, no GPU touched, status 2 (runtime failure)."""
    monkeypatch.setenv("AQ_FAULT_INJECT", "launch")
    assert _qp(lib) == _lib.AQ_ERUNTIME
    assert "injected" in _lib.last_error()
    assert _prod(lib, "aq_w4a16_gemv") == _lib.AQ_ERUNTIME
    assert _prod(lib, "aq_w4a16_gemm", M=128) == _lib.AQ_ERUNTIME
    assert _fp4(lib) == _lib.AQ_ERUNTIME
    assert _fp4q(lib) == _lib.AQ_ERUNTIME
    assert _qp(lib, "aq_quantize_pack_sym") == _lib.AQ_ERUNTIME
    assert _qp(lib, "aq_quantize_pack8") == _lib.AQ_ERUNTIME
    assert _prod8(lib, "aq_w8a16_gemv") == _lib.AQ_ERUNTIME
    assert _prod8(lib, "aq_w8a16_gemm", M=128) == _lib.AQ_ERUNTIME
    ws = lib.aq_act_absmean_workspace(64, 64)
    assert lib.aq_act_absmean(FAKE, 64, 64, FAKE, None, 64, FAKE, ws, None) == _lib.AQ_ERUNTIME
    assert lib.aq_awq_fold_norm(FAKE + 2, 1, FAKE, 64, FAKE, None) == _lib.AQ_ERUNTIME   # bf16: 2-byte aligned
    assert lib.aq_act_absmean_noalloc(FAKE, 64, 64, FAKE, None, 64, None) == _lib.AQ_ERUNTIME
    # validation still wins over the injected fault
    assert _qp(lib, g=5) == _lib.AQ_EINVAL


def test_status_mapping_in_python(lib):
    with pytest.raises(ValueError):
        _lib.check(_lib.AQ_EINVAL, "x")
    with pytest.raises(RuntimeError):
        _lib.check(_lib.AQ_ERUNTIME, "x")
    _lib.check(_lib.AQ_OK, "x")


def test_last_error_is_thread_local(lib):
    import threading
    assert _qp(lib, g=5) == _lib.AQ_EINVAL
    seen = {}

    def worker():
        seen["msg"] = ctypes.string_at(lib.aq_last_error()).decode() if lib.aq_last_error() else ""
    th = threading.Thread(target=worker)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "group" in _lib.last_error()
