"""GPU parity of the 8-bit variant: aq_quantize_pack8 (bit-exact codes, S, z) and the W8A16
GEMV / GEMM (tolerance, and bit-exact on an exactly representable case), through the C ABI,
against the CPU oracle (oracle.int4.quantize_codes8 / forward8)."""
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


def _assert_equal(got, want, what):
    (c, s, z), (c0, s0, z0) = got, want
    bad = (int(np.count_nonzero(c != c0)), int(np.count_nonzero(s.view(np.uint32) != s0.view(np.uint32))),
           int(np.count_nonzero(z != z0)))
    print(f"[gpu] {what}: mismatching codes {bad[0]}, scales {bad[1]}, zeros {bad[2]}", flush=True)
    assert bad == (0, 0, 0)


@pytest.mark.parametrize("g", [32, 64, 128])
def test_pack8_bit_exact(g):
    for name in ("gate_proj", "down_proj"):
        wb = synth.layer_weight_bf16(5, name)
        step(f"aq_quantize_pack8 {name} bf16 g={g}")
        got = tuple(host(t) for t in B.aq_quantize_pack8(dev_bf16(wb), g))
        _assert_equal(got, int4.quantize_codes8(synth.bf16_bits_to_f32(wb), g), f"pack8 {name} g={g}")
    rng = np.random.default_rng(g + 1)
    w = (rng.standard_normal((64, 384)) * 0.02).astype(np.float32)
    w[3, :g] = 0.125                                         # a constant group
    s = rng.uniform(0.25, 4.0, 384).astype(np.float32)
    step(f"aq_quantize_pack8 fp32 + channel scale g={g}")
    got = tuple(host(t) for t in B.aq_quantize_pack8(dev(w), g, dev(s)))
    _assert_equal(got, int4.quantize_codes8(w, g, s), f"pack8 fp32 scaled g={g}")


def _layer8(seed, name, g):
    return int4.quantize_codes8(synth.bf16_bits_to_f32(synth.layer_weight_bf16(seed, name)), g)


@pytest.mark.parametrize("g", [64, 128])
def test_gemv8_decoder_layer(g):
    for name, n, k in synth.LAYER_LINEARS:
        c, s, z = _layer8(6, name, g)
        dc, ds, dz = dev(c), dev(s), dev(z)
        for m in (1, 4, 16):
            xb = synth.layer_activations_bf16(6, m, k)
            step(f"aq_w8a16_gemv {name} [{n},{k}] g={g} M={m}")
            y = host(B.aq_w8a16_gemv(dev_bf16(xb), dc, ds, dz, g))
            check_close(y, int4.forward8(synth.bf16_bits_to_f32(xb), c, s, z, g), f"gemv8 {name} g={g} M={m}")


@pytest.mark.parametrize("m,name", [(64, "q_proj"), (300, "k_proj"), (2048, "gate_proj"), (17, "down_proj")])
def test_gemm8_shapes(m, name):
    c, s, z = _layer8(7, name, 64)
    n, k = synth.LINEAR_SHAPES[name]
    xb = synth.layer_activations_bf16(7, m, k)
    step(f"aq_w8a16_gemm {name} [{n},{k}] M={m}")
    y = host(B.aq_w8a16_gemm(dev_bf16(xb), dev(c), dev(s), dev(z), 64))
    check_close(y, int4.forward8(synth.bf16_bits_to_f32(xb), c, s, z, 64), f"gemm8 {name} M={m}")


@pytest.mark.parametrize("m,n,k,g", [(1, 64, 256, 64), (5, 33, 512, 32), (16, 130, 1024, 128), (70, 130, 512, 64),
                                     (300, 200, 768, 128), (1, 1003, 512, 64), (4, 1001, 2048, 128),
                                     (2, 1002, 4096, 32), (12, 1001, 4160, 32), (8, 8197, 2048, 64),
                                     (16, 17, 64, 64), (5, 1001, 6272, 128), (16, 257, 8256, 64),
                                     (1, 1001, 2048, 64), (3, 130, 1536, 32), (6, 33, 4096, 128),
                                     (9, 40, 8192, 32), (3, 40, 11008, 64), (2, 33, 16384, 128), (3, 17, 160, 32),
                                     (2, 5001, 2048, 64), (1, 4099, 1024, 128), (3, 2049, 2048, 32),
                                     (1, 8191, 2048, 64), (1, 4099, 14336, 64), (2, 4097, 8192, 32),
                                     (3, 4100, 14336, 128), (3, 2047, 11008, 64)])
def test_int8_exact_integer_case(m, n, k, g):
    """Integer X (|x| <= 16), random codes and zero points, S = 2^-6: every product and partial
    sum is exact in fp32, so the GEMV / GEMM output equals the fp64 reference bit for bit (from
    M = 4 the decode runs on the matrix cores, here also over several 4096-k chunks and a ragged
    tail chunk; from one to three rows the VALU launch with one row per wave below N = 4096,
    two up to N = 8192 and four beyond; longer rows with the activations staged beyond 64 KiB
    of LDS, two or one row per wave, or unstaged when the blocks would need two rounds on 256
    CUs; ragged N)."""
    rng = np.random.default_rng(m * 7 + n)
    x = rng.integers(-16, 17, (m, k)).astype(np.float32)
    c = rng.integers(0, 256, (n, k)).astype(np.uint8)
    z = rng.integers(0, 256, (n, k // g)).astype(np.uint8)
    s = np.full((n, k // g), 2.0 ** -6, dtype=np.float32)
    fn = B.aq_w8a16_gemv if m <= 16 else B.aq_w8a16_gemm
    step(f"int8 exact case M={m} N={n} K={k} g={g}")
    y = host(fn(dev_bf16(synth.f32_to_bf16_bits(x)), dev(c), dev(s), dev(z), g))
    ref = int4.forward8(x, c, s, z, g)
    assert np.array_equal(y.astype(np.float64), ref), float(np.abs(y - ref).max())
