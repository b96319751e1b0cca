"""GPU parity: INT4 quantize/pack (bit-exact) and the W4A16 GEMV / GEMM (tolerance, and
bit-exact on an exactly representable case), through the C ABI, against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import int4
from tests.gpu_util import check_close, dev, dev_bf16, host, step
from weight_only_bit_group_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_only_bit_group_amd import binding
    globals()["B"] = binding


def _pack_gpu(w_dev, g, s_dev=None):
    p, s, z = B.aq_quantize_pack(w_dev, g, s_dev)
    return host(p), host(s), host(z)


def _assert_pack_equal(got, want, what):
    (p, s, z), (p0, s0, z0) = got, want
    bad_p = int(np.count_nonzero(p != p0))
    bad_s = int(np.count_nonzero(s.view(np.uint32) != s0.view(np.uint32)))
    bad_z = int(np.count_nonzero(z != z0))
    print(f"[gpu] {what}: mismatching packed bytes {bad_p}, scales {bad_s}, zeros {bad_z}", flush=True)
    assert bad_p == 0 and bad_s == 0 and bad_z == 0


# ---------------------------------------------------------------- quantize / pack

def test_pack_single_linear_fp32():
    case = synth.single_linear(0)
    step("aq_quantize_pack fp32 256x256 g=128")
    got = _pack_gpu(dev(case["W"]), 128)
    _assert_pack_equal(got, int4.quantize_pack(case["W"], 128), "single linear")


@pytest.mark.parametrize("g", [64, 128])
def test_pack_decoder_layer_bf16(g):
    for name, n, k in synth.LAYER_LINEARS:
        wb = synth.layer_weight_bf16(1, name)
        step(f"aq_quantize_pack bf16 {name} [{n},{k}] g={g}")
        got = _pack_gpu(dev_bf16(wb), g)
        _assert_pack_equal(got, int4.quantize_pack(synth.bf16_bits_to_f32(wb), g), f"{name} g={g}")


def _edge_matrix(rng, n, k, g):
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    vg = w.reshape(n, k // g, g)
    vg[0, 0] = 0.25                                   # constant group
    if vg.shape[1] > 1:
        vg[0, 1] = np.abs(vg[0, 1]) + 1.0             # all positive (z clamps to 0)
    if n > 1:
        vg[1, 0] = -np.abs(vg[1, 0]) - 1.0            # all negative (z clamps to 15)
    if n > 2:                                         # half-integer ties with odd zero point
        vg[2, 0] = (rng.integers(-10, 21, g) * 0.5).astype(np.float32)
        vg[2, 0, 0], vg[2, 0, 1] = -5.0, 10.0
    if n > 3:
        vg[3, 0] = 0.0                                # all-zero group
        vg[3, -1] *= np.float32(1e-30)                # tiny range
    if n > 5:                                         # range of one ulp: |v / S| ~ 1.3e8 > 2^22,
        one_up = np.nextafter(np.float32(1.0), np.float32(2.0))   # codes clamp to 15 / 0
        vg[4, 0] = np.where(np.arange(g) % 3 == 0, one_up, np.float32(1.0))
        vg[5, 0] = -vg[4, 0]
    return w


@pytest.mark.parametrize("n,k,g", [(1, 32, 32), (3, 64, 32), (37, 192, 64), (5, 384, 128), (257, 128, 64)])
def test_pack_edge_cases(n, k, g):
    rng = np.random.default_rng(n * 1000 + k + g)
    w = _edge_matrix(rng, n, k, g)
    step(f"aq_quantize_pack edge fp32 [{n},{k}] g={g}")
    _assert_pack_equal(_pack_gpu(dev(w), g), int4.quantize_pack(w, g), f"edge fp32 [{n},{k}] g={g}")
    wb = synth.f32_to_bf16_bits(w)
    step(f"aq_quantize_pack edge bf16 [{n},{k}] g={g}")
    _assert_pack_equal(_pack_gpu(dev_bf16(wb), g), int4.quantize_pack(synth.bf16_bits_to_f32(wb), g),
                       f"edge bf16 [{n},{k}] g={g}")


@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_pack_with_channel_scale(wdtype):
    rng = np.random.default_rng(7)
    n, k, g = 96, 512, 64
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    s = np.exp(rng.standard_normal(k) * 0.7).astype(np.float32)
    if wdtype == "bf16":
        wb = synth.f32_to_bf16_bits(w)
        w = synth.bf16_bits_to_f32(wb)
        wd = dev_bf16(wb)
    else:
        wd = dev(w)
    step(f"aq_quantize_pack with chan_scale {wdtype} [{n},{k}]")
    _assert_pack_equal(_pack_gpu(wd, g, dev(s)), int4.quantize_pack(w, g, s), f"scaled {wdtype}")


# ---------------------------------------------------------------- GEMV

def _quantized_layer(seed, name, g):
    wb = synth.layer_weight_bf16(seed, name)
    p, s, z = int4.quantize_pack(synth.bf16_bits_to_f32(wb), g)
    return p, s, z


def test_gemv_single_linear():
    case = synth.single_linear(0)
    p, s, z = int4.quantize_pack(case["W"], 128)
    step("aq_w4a16_gemv 256x256 g=128 M=8")
    y = host(B.aq_w4a16_gemv(dev_bf16(case["X"]), dev(p), dev(s), dev(z), 128))
    check_close(y, int4.forward(synth.bf16_bits_to_f32(case["X"]), p, s, z, 128), "gemv single linear M=8")


@pytest.mark.parametrize("g", [64, 128])
def test_gemv_decoder_layer(g):
    for name, n, k in synth.LAYER_LINEARS:
        p, s, z = _quantized_layer(2, name, g)
        dp, ds, dz = dev(p), dev(s), dev(z)
        for m in (1, 4, 16):
            xb = synth.layer_activations_bf16(2, m, k)
            step(f"aq_w4a16_gemv {name} [{n},{k}] g={g} M={m}")
            y = host(B.aq_w4a16_gemv(dev_bf16(xb), dp, ds, dz, g))
            check_close(y, int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, g), f"gemv {name} g={g} M={m}")


def _exact_case(rng, m, n, k, g):
    """Integer X (|x| <= 64) and S = 2^-6: every product and partial sum is exact in fp32."""
    x = rng.integers(-64, 65, (m, k)).astype(np.float32)
    q = rng.integers(0, 16, (n, k)).astype(np.uint8)
    z = rng.integers(0, 16, (n, k // g)).astype(np.uint8)
    s = np.full((n, k // g), 2.0 ** -6, dtype=np.float32)
    return synth.f32_to_bf16_bits(x), x, int4.pack_nibbles(q), s, z


@pytest.mark.parametrize("m,n,k,g", [(1, 64, 256, 64), (5, 33, 128, 32), (16, 130, 1024, 128), (1, 8195, 256, 64),
                                     (1, 8197, 2048, 32), (8, 40, 4160, 64), (9, 33, 2080, 32), (12, 17, 4224, 128),
                                     (16, 300, 32, 32), (7, 8195, 1024, 128), (16, 70, 8256, 32),
                                     (8, 70, 8192, 128), (5, 33, 4096, 64), (12, 12500, 512, 64),
                                     (9, 8300, 2048, 128), (8, 8192, 2048, 32), (5, 8250, 2048, 64),
                                     (4, 8200, 2048, 64), (3, 257, 2048, 64), (4, 500, 2048, 128),
                                     (1, 511, 2048, 32), (3, 130, 16384, 64), (4, 1001, 11008, 128),
                                     (2, 4097, 14336, 32), (3, 2049, 11008, 64), (2, 2047, 14336, 64),
                                     (1, 4097, 14336, 64), (1, 2047, 12416, 128), (1, 1001, 12288, 64)])
def test_gemv_exact_integer_case(m, n, k, g):
    """(N >= 8192 at M = 1 takes the four-rows-per-wave launch, here with a ragged last wave;
    N <= 512 the one-row-per-wave launch (the compile-time K = 2048 instance, ragged N);
    rows longer than 4096 codes at M = 2..4 the launch with the activations staged beyond
    64 KiB of LDS, or, when its blocks would not fit one round on 256 CUs, the previous one;
    rows of more than 12288 codes at M = 1 the eight-wave blocks (12288 itself four waves);
    M >= 5 takes the matrix-core kernels: the chunked one with 4, 8 and 16 waves per block,
    over several 4096-k chunks, a ragged tail chunk and a single group; from M = 8 at
    N >= 8192 and K <= 2048 the LDS-staged one, with 48 and 64 rows per block.)"""
    xb, x, p, s, z = _exact_case(np.random.default_rng(m + n + k), m, n, k, g)
    step(f"aq_w4a16_gemv exact-integer M={m} N={n} K={k} g={g}")
    y = host(B.aq_w4a16_gemv(dev_bf16(xb), dev(p), dev(s), dev(z), g))
    ref = int4.forward(x, p, s, z, g)
    assert (y.astype(np.float64) == ref).all()


@pytest.mark.parametrize("m,n,k,g", [(1, 1, 32, 32), (2, 7, 96, 32), (3, 4099, 320, 64), (16, 8200, 64, 64),
                                     (1, 8194, 512, 128), (1, 8199, 11008, 64), (8, 8197, 2048, 64),
                                     (13, 1001, 11008, 64), (10, 3, 6144, 128), (5, 8203, 1024, 64),
                                     (6, 8192, 256, 32), (2, 1003, 11008, 64), (3, 70, 8192, 32),
                                     (2, 8195, 2048, 64), (2, 9000, 1024, 128), (16, 13001, 1024, 32),
                                     (11, 8191, 2048, 64)])
def test_gemv_ragged_shapes(m, n, k, g):
    rng = np.random.default_rng(n)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    p, s, z = int4.quantize_pack(w, g)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    step(f"aq_w4a16_gemv ragged M={m} N={n} K={k} g={g}")
    y = host(B.aq_w4a16_gemv(dev_bf16(xb), dev(p), dev(s), dev(z), g))
    check_close(y, int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, g), f"gemv ragged {m}x{n}x{k}")


# ---------------------------------------------------------------- GEMM

def test_gemm_single_linear():
    case = synth.single_linear(0)
    p, s, z = int4.quantize_pack(case["W"], 128)
    step("aq_w4a16_gemm 256x256 g=128 M=8")
    y = host(B.aq_w4a16_gemm(dev_bf16(case["X"]), dev(p), dev(s), dev(z), 128))
    check_close(y, int4.forward(synth.bf16_bits_to_f32(case["X"]), p, s, z, 128), "gemm single linear M=8")


def test_gemm_prefill_layer_m512():
    for name, n, k in synth.LAYER_LINEARS:
        p, s, z = _quantized_layer(3, name, 64)
        xb = synth.layer_activations_bf16(3, 512, k)
        step(f"aq_w4a16_gemm {name} [{n},{k}] g=64 M=512")
        y = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), 64))
        check_close(y, int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, 64), f"gemm {name} M=512")


def test_gemm_prefill_gate_m4096_all_rows():
    """The metric shape (M=4096, K=2048, N=11008, g=64) in the benchmarked launch configuration
    (staged path, persistent grid): every output against the fp64 oracle, and the worst 256-row
    tile band on its own, so an error confined to one tile of the schedule cannot hide in the
    whole-matrix mean."""
    p, s, z = _quantized_layer(3, "gate_proj", 64)
    xb = synth.layer_activations_bf16(3, 4096, 2048)
    step("aq_w4a16_gemm gate_proj [11008,2048] g=64 M=4096")
    y = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), 64))
    ref = int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, 64)
    check_close(y, ref, "gemm gate M=4096 (all rows)")
    band = np.abs(y - ref).reshape(16, 256, -1).mean(axis=(1, 2))
    worst = int(band.argmax())
    check_close(y[256 * worst:256 * (worst + 1)], ref[256 * worst:256 * (worst + 1)],
                f"gemm gate M=4096 (rows {256 * worst}..{256 * worst + 255}, worst band)")


@pytest.mark.parametrize("m,n,k,g", [(1, 5, 64, 32), (64, 128, 128, 64), (300, 200, 192, 64), (257, 129, 384, 128),
                                     (2049, 130, 96, 32)])
def test_gemm_ragged_shapes(m, n, k, g):
    rng = np.random.default_rng(m * 7 + n)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    p, s, z = int4.quantize_pack(w, g)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    step(f"aq_w4a16_gemm ragged M={m} N={n} K={k} g={g}")
    y = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), g))
    check_close(y, int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, g), f"gemm ragged {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k,g", [(64, 128, 256, 64), (300, 130, 128, 32), (2100, 256, 512, 128)])
def test_gemm_exact_integer_case(m, n, k, g):
    xb, x, p, s, z = _exact_case(np.random.default_rng(m + n), m, n, k, g)
    step(f"aq_w4a16_gemm exact-integer M={m} N={n} K={k} g={g}")
    y = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), g))
    assert (y.astype(np.float64) == int4.forward(x, p, s, z, g)).all()


@pytest.mark.parametrize("m,n,k,g", [(2048, 130, 96, 32), (2300, 257, 2080, 32), (3072, 384, 640, 128),
                                     (2049, 257, 2112, 64), (4097, 129, 256, 64), (2100, 200, 32, 32)])
def test_gemm_staged_equals_fused(m, n, k, g):
    """The staged path (weights dequantized once into the workspace) and the fused path give
    bit-identical outputs: the same exact bf16 operands, MFMA order and group rescales.  The
    staged output is also checked against the oracle (ragged M and N, tail stages, K = 32)."""
    rng = np.random.default_rng(m + 3 * n + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    p, s, z = int4.quantize_pack(w, g)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    assert B.aq_w4a16_gemm_workspace(m, n, k, g) >= n * k * 2
    step(f"aq_w4a16_gemm staged M={m} N={n} K={k} g={g}")
    # exactly the staging matrix: the staged path without K slices
    ys = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), g,
                              workspace=torch.empty(n * k * 2, dtype=torch.uint8, device="cuda")))
    step(f"aq_w4a16_gemm fused M={m} N={n} K={k} g={g}")
    yf = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), g,
                              workspace=torch.empty(0, dtype=torch.uint8, device="cuda")))
    assert np.array_equal(ys.view(np.uint32), yf.view(np.uint32))
    check_close(ys, int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, g), f"gemm staged {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k,g", [(512, 2048, 2048, 64), (512, 256, 2048, 64), (300, 130, 4096, 128),
                                     (64, 8195, 2048, 32), (512, 2048, 11008, 64), (4096, 256, 2048, 64)])
def test_gemm_k_slices(m, n, k, g):
    """Few output tiles: K split into slices whose fp32 partials are added in order (with the
    staging matrix at M = 4096), against the oracle and the unsplit fused GEMM."""
    rng = np.random.default_rng(m + 5 * n + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    p, s, z = int4.quantize_pack(w, g)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    staged = n * k * 2 if m >= 2048 else 0
    need = B.aq_w4a16_gemm_workspace(m, n, k, g)
    assert need > staged and (need - ((staged + 255) // 256 * 256 if staged else 0)) % (m * n * 4) == 0
    step(f"aq_w4a16_gemm K slices M={m} N={n} K={k} g={g}")
    y = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), g,
                             workspace=torch.empty(need, dtype=torch.uint8, device="cuda")))
    step(f"aq_w4a16_gemm fused, no slices M={m} N={n} K={k} g={g}")
    yf = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), g,
                              workspace=torch.empty(0, dtype=torch.uint8, device="cuda")))
    assert np.abs(y - yf).max() <= 1e-5 * np.abs(yf).max()
    check_close(y, int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, g), f"gemm K slices {m}x{n}x{k}")


def test_gemm_k_slices_exact_integer_case():
    """Small integers: every partial and the ordered sum of the slices are exact in fp32."""
    m, n, k, g = 200, 130, 1024, 64
    xb, x, p, s, z = _exact_case(np.random.default_rng(17), m, n, k, g)
    assert B.aq_w4a16_gemm_workspace(m, n, k, g) > 0
    step(f"aq_w4a16_gemm K slices exact-integer M={m} N={n} K={k} g={g}")
    y = host(B.aq_w4a16_gemm(dev_bf16(xb), dev(p), dev(s), dev(z), g))
    assert (y.astype(np.float64) == int4.forward(x, p, s, z, g)).all()


def test_pack_then_gemv_round_trip():
    """Device pack followed by the device GEMV equals the oracle's pack + forward (the module-swap path)."""
    wb = synth.layer_weight_bf16(4, "o_proj")
    xb = synth.layer_activations_bf16(4, 1, 2048)
    step("aq_quantize_pack + aq_w4a16_gemv o_proj")
    p, s, z = B.aq_quantize_pack(dev_bf16(wb), 64)
    y = host(B.aq_w4a16_gemv(dev_bf16(xb), p, s, z, 64))
    p0, s0, z0 = int4.quantize_pack(synth.bf16_bits_to_f32(wb), 64)
    check_close(y, int4.forward(synth.bf16_bits_to_f32(xb), p0, s0, z0, 64), "pack+gemv o_proj")


def test_gemv_batch_in_a_hip_graph():
    """The decode GEMV allocates nothing and synchronizes nothing, so a batch of launches can
    be captured in a HIP graph (the bench times its decode batch that way).  Every replay,
    with eager work and synchronizations between replays, equals the eager result bit for bit."""
    ws = [synth.layer_weight_bf16(20 + i, "o_proj") for i in range(3)]
    xb = synth.layer_activations_bf16(7, 1, 2048)
    step("aq_w4a16_gemv x3 captured in a HIP graph")
    x = dev_bf16(xb)
    packs = [B.aq_quantize_pack(dev_bf16(w), 64) for w in ws]
    outs = [torch.empty((1, 2048), dtype=torch.float32, device=x.device) for _ in packs]

    def batch():
        for (p, s, z), y in zip(packs, outs):
            B.aq_w4a16_gemv(x, p, s, z, 64, out=y)

    batch()
    eager = [host(y).copy() for y in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        batch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        batch()
    torch.cuda.synchronize()
    other = B.aq_w4a16_gemv(dev_bf16(synth.layer_activations_bf16(8, 1, 2048)), *packs[0], 64)
    for rep in range(3):
        for y in outs:
            y.fill_(float("nan"))
        graph.replay()
        got = [host(y) for y in outs]
        for i, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {rep}, launch {i}"
        B.aq_w4a16_gemv(x, *packs[1], 64, out=other)   # eager work between replays
        torch.cuda.synchronize()
    check_close(eager[0], int4.forward(synth.bf16_bits_to_f32(xb), *int4.quantize_pack(
        synth.bf16_bits_to_f32(ws[0]), 64), 64), "graph gemv o_proj")


# ---------------------------------------------------------------- symmetric variant

@pytest.mark.parametrize("g", [32, 64, 128])
def test_pack_sym_decoder_layer_bit_exact(g):
    """aq_quantize_pack_sym: codes, S and z bit-exact against the oracle on the layer's linears
    (bf16) and on fp32 weights with an AWQ channel scale and all-zero groups."""
    for name in ("q_proj", "down_proj"):
        wb = synth.layer_weight_bf16(3, name)
        step(f"aq_quantize_pack_sym {name} bf16 g={g}")
        got = tuple(host(t) for t in B.aq_quantize_pack(dev_bf16(wb), g, sym=True))
        _assert_pack_equal(got, int4.quantize_pack_sym(synth.bf16_bits_to_f32(wb), g), f"sym pack {name} g={g}")
    rng = np.random.default_rng(g)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    w[5, :g] = 0.0
    s = rng.uniform(0.25, 4.0, 512).astype(np.float32)
    step(f"aq_quantize_pack_sym fp32 + channel scale g={g}")
    got = tuple(host(t) for t in B.aq_quantize_pack(dev(w), g, dev(s), sym=True))
    _assert_pack_equal(got, int4.quantize_pack_sym(w, g, s), f"sym pack fp32 scaled g={g}")


@pytest.mark.parametrize("m", [1, 16, 300])
def test_sym_packs_through_gemv_and_gemm(m):
    """The symmetric packs decode with the unchanged GEMV (M <= 16) / GEMM: within tolerance of
    the oracle's forward on the same triple."""
    wb = synth.layer_weight_bf16(4, "gate_proj")
    p, s, z = int4.quantize_pack_sym(synth.bf16_bits_to_f32(wb), 64)
    xb = synth.layer_activations_bf16(4, m, 2048)
    step(f"sym gate_proj forward M={m}")
    fn = B.aq_w4a16_gemv if m <= 16 else B.aq_w4a16_gemm
    y = host(fn(dev_bf16(xb), dev(p), dev(s), dev(z), 64))
    check_close(y, int4.forward(synth.bf16_bits_to_f32(xb), p, s, z, 64), f"sym forward M={m}")
