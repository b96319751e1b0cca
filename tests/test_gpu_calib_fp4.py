"""GPU parity: activation abs-mean (bit-exact mean), AWQ alpha search (bit-exact alpha, scale
and packed triple), and the FP4 decode GEMV / GEMM (tolerance, and bit-exact on an exactly
representable case), through the C ABI, against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import awq, fp4, int4, stats
from tests.gpu_util import check_close, dev, dev_bf16, host, step
from weight_only_bit_group_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_only_bit_group_amd import binding
    globals()["B"] = binding


def _ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))


# ---------------------------------------------------------------- abs-mean

def _absmean_gpu(xb, count=None, sum_dev=None):
    x = dev_bf16(xb)
    t, k = xb.shape
    if sum_dev is None:
        sum_dev = torch.zeros(k, dtype=torch.float64, device="cuda")
    mean = torch.empty(k, dtype=torch.float32, device="cuda")
    B.aq_act_absmean(x, sum_dev, count or t, mean)
    return sum_dev, mean


def test_absmean_calibration_full():
    """128 samples x 512 tokens x 2048 channels, heavy-tailed channel magnitudes."""
    xb = synth.calibration_bf16(4)
    step("aq_act_absmean [65536, 2048]")
    s, m = _absmean_gpu(xb)
    s, m = host(s), host(m)
    x = synth.bf16_bits_to_f32(xb)
    ref_sum = stats.abs_sum(x)
    ref_m = stats.mean_from_sum(ref_sum, x.shape[0])
    u = _ulps(m, ref_m)
    print(f"[gpu] absmean: mean mismatches {int((u != 0).sum())} (max ulp {int(u.max())}), "
          f"sum mismatches {int((s != ref_sum).sum())}", flush=True)
    assert (m.view(np.uint32) == ref_m.view(np.uint32)).all()
    assert np.allclose(s, ref_sum, rtol=1e-15, atol=0)


@pytest.mark.parametrize("t,k", [(1, 8), (3, 520), (1000, 136), (4099, 2048)])
def test_absmean_ragged(t, k):
    xb = synth.calibration_rows_bf16(t + k, t, k)
    step(f"aq_act_absmean ragged [{t},{k}]")
    s, m = _absmean_gpu(xb)
    x = synth.bf16_bits_to_f32(xb)
    assert (host(m).view(np.uint32) == stats.absmean(x).view(np.uint32)).all()
    assert np.allclose(host(s), stats.abs_sum(x), rtol=1e-15, atol=0)


def test_absmean_accumulates_chunks():
    """Two chunks fed one after the other equal the whole (the merge of calibration runs)."""
    xb = synth.calibration_rows_bf16(9, 3000, 512)
    step("aq_act_absmean chunked 1200 + 1800 rows")
    s = torch.zeros(512, dtype=torch.float64, device="cuda")
    _absmean_gpu(xb[:1200], 1200, s)
    _, m = _absmean_gpu(xb[1200:], 3000, s)
    x = synth.bf16_bits_to_f32(xb)
    ref = stats.mean_from_sum(stats.abs_sum(x[:1200]) + stats.abs_sum(x[1200:]), 3000)
    assert (host(m).view(np.uint32) == ref.view(np.uint32)).all()


# ---------------------------------------------------------------- AWQ search

def _search_case(seed, t, n, k, wname=None):
    xb = synth.calibration_rows_bf16(seed, t, k)
    x = synth.bf16_bits_to_f32(xb)
    m = stats.absmean(x)
    if wname is None:
        rng = np.random.default_rng(seed + 1)
        wb = synth.f32_to_bf16_bits(synth.weight_f32(rng, n, k, 0.02, outlier_frac=0.001))
    else:
        wb = synth.layer_weight_bf16(seed, wname)
    return xb, x, m, wb


def _check_search(res, ref, what):
    mse = host(res["mse"])
    best = int(host(res["best"])[0])
    order = np.argsort(ref["mse"])
    gap = (ref["mse"][order[1]] - ref["mse"][order[0]]) / ref["mse"][order[0]]
    rel = np.abs(mse - ref["mse"]) / ref["mse"]
    print(f"[gpu] {what}: best gpu {best} oracle {ref['best']}; best-vs-second gap {gap:.3e}; "
          f"max mse rel err {rel.max():.3e}", flush=True)
    assert rel.max() < 1e-4
    assert best == ref["best"]
    assert (host(res["best_scale"]).view(np.uint32) == ref["scale"].view(np.uint32)).all()
    assert (host(res["packed"]) == ref["packed"]).all()
    assert (host(res["scales"]).view(np.uint32) == ref["scales"].view(np.uint32)).all()
    assert (host(res["zeros"]) == ref["zeros"]).all()


@pytest.mark.parametrize("t,n,k,g", [(256, 96, 256, 64), (300, 130, 384, 128), (64, 40, 128, 32)])
def test_search_small(t, n, k, g):
    xb, x, m, wb = _search_case(t + n, t, n, k)
    w = synth.bf16_bits_to_f32(wb)
    step(f"aq_awq_search T={t} N={n} K={k} g={g}")
    res = B.aq_awq_search(dev_bf16(xb), m, dev_bf16(wb), g, 20)
    _check_search(res, awq.search(x, m, w, g, 20), f"search {t}x{n}x{k}")


@pytest.mark.parametrize("t,n,k,g", [(520, 200, 256, 32), (300, 130, 128, 64), (1000, 17, 96, 32),
                                     (700, 300, 320, 64), (129, 257, 128, 128)])
def test_search_gram_form(t, n, k, g):
    """T > K: the MSE numerator through H = X^T X (ragged T padded to 64, ragged N and K tiles, the
    32-wide last stage at K = 96), against the oracle's direct (X E^T)^2."""
    xb, x, m, wb = _search_case(t + n + k, t, n, k)
    w = synth.bf16_bits_to_f32(wb)
    step(f"aq_awq_search Gram T={t} N={n} K={k} g={g}")
    res = B.aq_awq_search(dev_bf16(xb), m, dev_bf16(wb), g, 20)
    _check_search(res, awq.search(x, m, w, g, 20), f"search Gram {t}x{n}x{k}")


def test_search_gram_form_correlated_channels():
    """A strong common component across channels (large off-diagonal H): the Gram form keeps the
    alpha choice and the MSE."""
    t, n, k, g = 512, 96, 256, 64
    rng = np.random.default_rng(77)
    x = synth.bf16_bits_to_f32(synth.calibration_rows_bf16(77, t, k)).astype(np.float64)
    x += np.outer(rng.standard_normal(t) * 30.0, np.exp(1.5 * rng.standard_normal(k)))
    xb = synth.f32_to_bf16_bits(x.astype(np.float32))
    x = synth.bf16_bits_to_f32(xb)
    m = stats.absmean(x)
    wb = synth.f32_to_bf16_bits(synth.weight_f32(rng, n, k, 0.02, outlier_frac=0.001))
    step(f"aq_awq_search Gram correlated T={t} N={n} K={k}")
    res = B.aq_awq_search(dev_bf16(xb), m, dev_bf16(wb), g, 20)
    _check_search(res, awq.search(x, m, synth.bf16_bits_to_f32(wb), g, 20), "search Gram correlated")


def test_search_alpha_zero_only_equals_plain_pack():
    """n_grid = 1 is the alpha = 0 candidate only: s = 1 and the pack equals plain min-max."""
    xb, x, m, wb = _search_case(5, 128, 64, 256)
    step("aq_awq_search n_grid=1")
    res = B.aq_awq_search(dev_bf16(xb), m, dev_bf16(wb), 64, 1)
    assert int(host(res["best"])[0]) == 0
    assert (host(res["best_scale"]) == 1).all()
    p, s, z = int4.quantize_pack(synth.bf16_bits_to_f32(wb), 64)
    assert (host(res["packed"]) == p).all() and (host(res["zeros"]) == z).all()
    assert (host(res["scales"]).view(np.uint32) == s.view(np.uint32)).all()


@pytest.mark.parametrize("wname", ["q_proj", "gate_proj"])
def test_search_calibration_layer(wname):
    """Full size: 4096 calibration tokens (the first rows of the 128 x 512 set), g = 64, 20 alphas."""
    xb_full = synth.calibration_bf16(4)
    m = stats.absmean(synth.bf16_bits_to_f32(xb_full))
    xb = np.ascontiguousarray(xb_full[:4096])
    del xb_full
    wb = synth.layer_weight_bf16(4, wname)
    step(f"aq_awq_search {wname} T=4096 g=64")
    res = B.aq_awq_search(dev_bf16(xb), m, dev_bf16(wb), 64, 20)
    ref = awq.search(synth.bf16_bits_to_f32(xb), m, synth.bf16_bits_to_f32(wb), 64, 20)
    _check_search(res, ref, f"search {wname}")


# ---------------------------------------------------------------- FP4

def _fp4_case(n, k, seed=5):
    w = synth.fp4_weight_f32(seed, n, k)
    return fp4.encode(w)


@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
def test_fp4_mlp_shapes(n, k):
    c, b, ts = _fp4_case(n, k)
    dc, db = dev(c), dev(b)
    x1 = synth.layer_activations_bf16(5, 1, k)
    step(f"aq_fp4_gemm [{n},{k}] M=1")
    y = host(B.aq_fp4_gemm(dev_bf16(x1), dc, db, ts))
    check_close(y, fp4.forward(synth.bf16_bits_to_f32(x1), c, b, ts), f"fp4 [{n},{k}] M=1")
    x2 = synth.layer_activations_bf16(5, 2048, k)
    step(f"aq_fp4_gemm [{n},{k}] M=2048")
    y = host(B.aq_fp4_gemm(dev_bf16(x2), dc, db, ts))
    check_close(y, fp4.forward(synth.bf16_bits_to_f32(x2), c, b, ts), f"fp4 [{n},{k}] M=2048 (all rows)")


@pytest.mark.parametrize("m,n,k", [(1, 3, 32), (7, 130, 96), (16, 4100, 64), (17, 33, 160), (300, 257, 512),
                                   (1, 8195, 4096), (2, 4099, 160), (8, 8195, 4096), (12, 33, 2112), (4, 130, 64),
                                   (6, 70, 8256), (16, 9000, 2048), (3, 1001, 4160),
                                   (1, 4099, 160), (1, 130, 4160), (1, 70, 14368), (5, 40, 8192),
                                   (11, 17, 4096), (13, 12400, 512), (12, 8192, 2048), (16, 8193, 64),
                                   (4, 8200, 2048), (2, 70, 16384), (2, 130, 16416), (1, 33, 32768)])
def test_fp4_ragged(m, n, k):
    rng = np.random.default_rng(m + n + k)
    c, b, ts = fp4.encode((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    step(f"aq_fp4_gemm ragged M={m} N={n} K={k}")
    y = host(B.aq_fp4_gemm(dev_bf16(xb), dev(c), dev(b), ts))
    check_close(y, fp4.forward(synth.bf16_bits_to_f32(xb), c, b, ts), f"fp4 ragged {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(2048, 130, 96), (2048, 257, 512), (2100, 4100, 64)])
def test_fp4_staged_equals_fused(m, n, k):
    """FP4 GEMM: staged (exact bf16 weights in the workspace) and fused paths are bit-identical and
    match the oracle."""
    rng = np.random.default_rng(m + n + k + 1)
    c, b, ts = fp4.encode((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    assert B.aq_fp4_gemm_workspace(m, n, k) == n * k * 2
    step(f"aq_fp4_gemm staged M={m} N={n} K={k}")
    ys = host(B.aq_fp4_gemm(dev_bf16(xb), dev(c), dev(b), ts))
    step(f"aq_fp4_gemm fused M={m} N={n} K={k}")
    yf = host(B.aq_fp4_gemm(dev_bf16(xb), dev(c), dev(b), ts, workspace=torch.empty(0, dtype=torch.uint8,
                                                                                  device="cuda")))
    assert np.array_equal(ys.view(np.uint32), yf.view(np.uint32))
    check_close(ys, fp4.forward(synth.bf16_bits_to_f32(xb), c, b, ts), f"fp4 staged {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 5, 16, 64, 300])
def test_fp4_exact_case(m):
    """Small-integer X, every E2M1 code, block scales in {1/8 .. 4} and ts = 1: every product and
    partial sum is exact in fp32, so Y equals the fp64 reference bit for bit."""
    rng = np.random.default_rng(m)
    n, k = 96, 256
    c = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
    b = rng.choice(np.array([0x20, 0x28, 0x30, 0x38, 0x40, 0x48], np.uint8), (n, k // 16))
    x = rng.integers(-8, 9, (m, k)).astype(np.float32)
    step(f"aq_fp4_gemm exact M={m}")
    y = host(B.aq_fp4_gemm(dev_bf16(synth.f32_to_bf16_bits(x)), dev(c), dev(b), 1.0))
    assert (y.astype(np.float64) == fp4.forward(x, c, b, np.float32(1.0))).all()


# ---------------------------------------------------------------- FP4 encoder

def _encode_gpu(w_dev):
    c, b, ts = B.aq_fp4_quantize(w_dev)
    return host(c), host(b), host(ts)[0]


def _assert_encoding_equal(got, want, what):
    (c, b, ts), (c0, b0, ts0) = got, want
    bad_c = int(np.count_nonzero(c != c0))
    bad_b = int(np.count_nonzero(b != b0))
    print(f"[gpu] {what}: ts {ts!r} vs {np.float32(ts0)!r}, mismatching code bytes {bad_c}, scale bytes {bad_b}",
          flush=True)
    assert np.float32(ts).view(np.uint32) == np.float32(ts0).view(np.uint32)
    assert bad_c == 0 and bad_b == 0


@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
def test_fp4_quantize_mlp_shapes_bit_exact(n, k):
    """aq_fp4_quantize reproduces the oracle encoder byte for byte on the 7B-like MLP shapes."""
    w = synth.fp4_weight_f32(5, n, k)
    step(f"aq_fp4_quantize fp32 [{n},{k}]")
    _assert_encoding_equal(_encode_gpu(dev(w)), fp4.encode(w), f"fp4 encode [{n},{k}]")


def _edge_weight():
    """ts = 1 exactly (max |w| = 2688) and blocks built to land on every rounding decision:
    E4M3 ties (block amax / 6 halfway between two codes, normal and subnormal), E4M3
    saturation, E2M1 midpoints of both parities, a value past 6, signed zeros, a zero block."""
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -5.0, 6.0, -6.0, -0.0, 0.0]
    # block amax 6.375: target 1.0625, halfway between E4M3 1.0 (even code) and 1.125 -> scale
    # 1, and 6.375 itself saturates to the largest E2M1 code
    rows.append([6.375] + mids)
    # block amax 6 * 2.5 / 512: target 2.5 * 2^-9 (subnormal tie) -> code 2, scale 2^-8
    sub = 6 * 2.5 / 512
    rows.append([sub] + [v * 2.0 ** -8 for v in mids])
    # block amax 2688: target 448 -> 0x7E, scale 448 (midpoints up to 5: nothing above 2688)
    small = [v for v in mids if abs(v) <= 5.0]
    rows.append([2688.0] + [v * 448 for v in small] + [0.0] * (15 - len(small)))
    # block amax 6 * 432: target 432, halfway between 416 and 448 -> 448 (even code)
    rows.append([6 * 432.0] + [v * 448 for v in small] + [0.0] * (15 - len(small)))
    # all-zero block and a block of tiny values
    rows.append([0.0] * 16)
    rows.append([1e-30 * (i + 1) * (-1) ** i for i in range(16)])
    rng = np.random.default_rng(9)
    w = np.array(rows, dtype=np.float32).reshape(-1)
    w = np.concatenate([w, (rng.standard_normal(16 * 58) * 3).astype(np.float32)])
    return w.reshape(4, -1)


def test_fp4_quantize_rounding_edges_bit_exact():
    w = _edge_weight()
    step(f"aq_fp4_quantize edge cases {w.shape}")
    want = fp4.encode(w)
    assert np.float32(want[2]) == np.float32(1.0)
    _assert_encoding_equal(_encode_gpu(dev(w)), want, "fp4 encode edges")


def test_fp4_quantize_bf16_input_and_all_zero():
    wb = synth.f32_to_bf16_bits(synth.fp4_weight_f32(6, 256, 512))
    step("aq_fp4_quantize bf16 [256,512]")
    _assert_encoding_equal(_encode_gpu(dev_bf16(wb)), fp4.encode(synth.bf16_bits_to_f32(wb)), "fp4 encode bf16")
    z = np.zeros((8, 64), np.float32)
    step("aq_fp4_quantize all-zero [8,64]")
    c, b, ts = _encode_gpu(dev(z))
    assert ts == np.float32(1.0) and not c.any() and not b.any()


def test_fp4_quantize_then_decode_product():
    """Encode on the GPU, then run the FP4 GEMV / GEMM on its output: equal to the oracle's
    decode of the oracle's encoding (the same bytes), within the product tolerance."""
    w = synth.fp4_weight_f32(7, 1024, 2048)
    xb = synth.layer_activations_bf16(7, 64, 2048)
    step("aq_fp4_quantize + aq_fp4_gemm [1024,2048] M=64")
    c, b, ts = B.aq_fp4_quantize(dev(w))
    y = host(B.aq_fp4_gemm(dev_bf16(xb), c, b, float(host(ts)[0])))
    c0, b0, ts0 = fp4.encode(w)
    check_close(y, fp4.forward(synth.bf16_bits_to_f32(xb), c0, b0, ts0), "fp4 encode + gemm")
