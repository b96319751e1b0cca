"""Pins of the FP4 (E2M1 codes, E4M3 per-16 block scales) oracle."""
import json
import os

import numpy as np

from oracle import fp4
from weight_only_bit_group_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_table():
    """The 8 E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 and bit 3 is the sign."""
    assert fp4.e2m1_value(np.arange(8)).tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert fp4.e2m1_value(np.arange(8, 16)).tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert fp4.e2m1_value(0b0111) == 6.0


def test_e4m3_bit_split_and_spot_values():
    """1 sign + 4 exponent + 3 mantissa bits (the FP8 section's split): spot values, the
    largest finite value, subnormals, NaN, and monotone ordering of the positive codes."""
    v = fp4.e4m3_value(np.arange(256))
    assert fp4.e4m3_value(0x7E) == 448.0
    assert fp4.e4m3_value(0x38) == 1.0
    assert fp4.e4m3_value(0x01) == 2.0 ** -9
    assert fp4.e4m3_value(0x08) == 2.0 ** -6
    assert fp4.e4m3_value(0x07) == 7 * 2.0 ** -9
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(np.delete(v, [0x7F, 0xFF])).all()
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()
    assert (v[0x80:0xFF] == -pos[:0x7F]).all()
    # each exponent step doubles the value; the 3 mantissa bits give 8 steps per binade
    assert all(fp4.e4m3_value(b + 8) == 2 * fp4.e4m3_value(b) for b in range(8, 0x76))


def test_products_exact_in_bf16():
    """P13: every E2M1 x E4M3 product (16 x 254 finite bytes) is exactly representable in bf16."""
    c = fp4.e2m1_value(np.arange(16))[:, None]
    b = np.delete(np.arange(256), [0x7F, 0xFF])
    p = (c * fp4.e4m3_value(b)[None, :]).astype(np.float32)
    back = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(p))
    assert (back == p).all()
    assert (p.astype(np.float64) == c * fp4.e4m3_value(b)[None, :]).all()


def test_e4m3_encode_rounding():
    """Nearest-even rounding and saturation of the block-scale encoder, checked against brute
    force over all finite codes."""
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.uniform(0, 500, 2000), fp4.e4m3_value(np.arange(0x7F)),
                        (fp4.e4m3_value(np.arange(0x7E)) + fp4.e4m3_value(np.arange(1, 0x7F))) / 2])
    codes = fp4.e4m3_encode(a)
    vals = fp4.e4m3_value(np.arange(0x7F))
    for x, c in zip(a, codes):
        d = np.abs(vals - min(x, 448.0))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want


def test_encoder_round_trip_bound():
    """Encoder (parity unpinned beyond this): |w - w_hat| <= half an E2M1 step at the block's
    scale, with the step taken at the magnitude of w (steps 0.5 below 2, 1 below 4, 2 above)."""
    w = synth.fp4_weight_f32(5, 64, 256)
    codes, b, ts = fp4.encode(w)
    what = fp4.dequantize(codes, b, ts)
    sc = np.repeat(fp4.e4m3_value(b), 16, axis=-1) * float(ts)
    r = np.abs(w) / sc
    step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    err = np.abs(w.astype(np.float64) - what)
    assert (err <= 0.5 * step * sc * (1 + 1e-6) + 1e-30).all()
    assert float(ts) == float(np.float32(np.abs(w).max() / np.float32(2688)))


def test_forward_matches_definition():
    """Y = X W_hat^T with W_hat = e2m1 * e4m3 * ts, against a per-element loop on a tiny case."""
    rng = np.random.default_rng(4)
    w = synth.fp4_weight_f32(6, 3, 32)
    codes, b, ts = fp4.encode(w)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((2, 32)).astype(np.float32)))
    y = fp4.forward(x, codes, b, ts)
    for i in range(2):
        for n in range(3):
            acc = 0.0
            for k in range(32):
                byte = int(codes[n, k // 2])
                code = (byte >> (4 * (k % 2))) & 0xF
                acc += float(x[i, k]) * float(fp4.e2m1_value(code)) * float(fp4.e4m3_value(b[n, k // 16])) * float(ts)
            assert abs(acc - y[i, n]) <= 1e-12 * max(1.0, abs(acc))


def test_golden_regression():
    with open(os.path.join(GOLDEN, "fp4_small.json")) as f:
        gold = json.load(f)
    codes, b, ts = fp4.encode(synth.fp4_weight_f32(5, 8, 64))
    assert codes.tobytes().hex() == gold["codes_hex"]
    assert b.tolist() == gold["block_scales"]
    assert int(np.float32(ts).view(np.uint32)) == gold["ts_bits"]
