"""Pins of the norm-group AWQ / fold / decoder-layer oracle (oracle/layer.py)."""
import math
import struct

import numpy as np
import pytest

from oracle import awq, int4, layer


def test_bf16_round_ties_to_even():
    one = np.float32(1.0)
    u = np.float32(2.0 ** -7)   # bf16 ulp at 1
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8)], np.float32)
    want = np.array([one, one + 2 * u, one + u, -one], np.float32)
    assert (layer.bf16_round(vals) == want).all()


def test_rms_norm_closed_form():
    d, c = 64, -0.75
    w = np.linspace(0.5, 1.5, d)
    got = layer.rms_norm(np.full((3, d), c), w)
    want = c / np.sqrt(c * c + layer.RMS_EPS) * w
    assert np.allclose(got, want[None, :], rtol=1e-15, atol=0)


def test_silu_odd_part_identity():
    x = np.linspace(-9, 9, 101)
    assert layer.silu(np.zeros(1))[0] == 0.0
    assert np.allclose(layer.silu(x) - layer.silu(-x), x, rtol=1e-14, atol=1e-14)


def test_attention_single_token_and_uniform_keys():
    """One token: the output is its value row (per grouped head).  Zero keys: softmax is
    uniform, so token t's output is the mean of the first t + 1 value rows."""
    rng = np.random.default_rng(0)
    nh, nkv, hd, t = 4, 2, 8, 5
    q = rng.standard_normal((t, nh * hd))
    v = rng.standard_normal((t, nkv * hd))
    one = layer.causal_attention(q[:1], rng.standard_normal((1, nkv * hd)), v[:1], nh, nkv)
    for h in range(nh):
        kv = h // (nh // nkv)
        assert np.allclose(one[0, h * hd:(h + 1) * hd], v[0, kv * hd:(kv + 1) * hd], rtol=1e-15)
    out = layer.causal_attention(q, np.zeros((t, nkv * hd)), v, nh, nkv)
    for i in range(t):
        for h in range(nh):
            kv = h // (nh // nkv)
            assert np.allclose(out[i, h * hd:(h + 1) * hd], v[:i + 1, kv * hd:(kv + 1) * hd].mean(axis=0), rtol=1e-13)


def test_attention_is_causal():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((6, 32)) for _ in range(3))
    a = layer.causal_attention(q, k, v, 2, 1)
    k2, v2 = k.copy(), v.copy()
    k2[4:] += 3.0
    v2[4:] -= 5.0
    b = layer.causal_attention(q, k2, v2, 2, 1)
    assert np.array_equal(a[:4], b[:4]) and not np.allclose(a[4:], b[4:])


def test_joint_mse_is_the_row_weighted_mean():
    """For one channel scale, the output MSE of the concatenated consumers is the N-weighted
    mean of their own MSEs (the joint search scores T x (N1 + N2) elements)."""
    rng = np.random.default_rng(2)
    k, g = 128, 64
    x = rng.standard_normal((16, k)).astype(np.float32)
    w1 = (rng.standard_normal((24, k)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((8, k)) * 0.02).astype(np.float32)
    s = awq.candidate_scale(np.abs(x).mean(axis=0), 0.35)
    m1 = awq.output_mse(x, awq.error_matrix(w1, g, s))
    m2 = awq.output_mse(x, awq.error_matrix(w2, g, s))
    mj = awq.output_mse(x, awq.error_matrix(np.concatenate([w1, w2]), g, s))
    assert abs(mj - (24 * m1 + 8 * m2) / 32) <= 1e-12 * mj


def test_fold_direction_is_exact_for_power_of_two_scales():
    """rms_norm(h, w / s) (s W)^T equals rms_norm(h, w) W^T bit for bit when every s_k is a
    power of two: the fold divides the norm weight by the scale that multiplies W."""
    rng = np.random.default_rng(3)
    k = 64
    h = rng.standard_normal((5, k))
    w_norm = rng.uniform(0.5, 1.5, k).astype(np.float32)
    wm = (rng.standard_normal((12, k)) * 0.02).astype(np.float32)
    s = np.float32(2.0) ** rng.integers(-3, 4, k).astype(np.float32)
    folded = (w_norm / s).astype(np.float32)
    lhs = layer.rms_norm(h, folded) @ (wm.astype(np.float64) * s).T
    rhs = layer.rms_norm(h, w_norm) @ wm.astype(np.float64).T
    assert np.array_equal(lhs, rhs)


def test_norm_group_split_equals_per_matrix_pack():
    """The joint result's per-matrix triples are each matrix packed with the common scale
    (packing is row-wise, so concatenating and splitting commute)."""
    rng = np.random.default_rng(4)
    k, g = 128, 64
    x = rng.standard_normal((32, k)).astype(np.float32) * rng.uniform(0.1, 3, k).astype(np.float32)
    ws = [(rng.standard_normal((n, k)) * 0.02).astype(np.float32) for n in (16, 8, 8)]
    r = layer.norm_group_awq(x, np.ones(k, np.float32), ws, g, n_grid=5)
    for w, (p, sc, z) in zip(ws, r["packs"]):
        p0, s0, z0 = int4.quantize_pack(w, g, r["search"]["scale"])
        assert np.array_equal(p, p0) and np.array_equal(sc, s0) and np.array_equal(z, z0)
    assert np.array_equal(r["norm"], (np.ones(k, np.float32) / r["search"]["scale"]).astype(np.float32))


def test_layer_with_zero_output_projections_is_identity():
    """o_proj = down_proj = 0: both residual branches vanish and the layer returns h."""
    rng = np.random.default_rng(5)
    d, nh, nkv, hd, inter = 64, 2, 1, 32, 96
    h = rng.standard_normal((4, d))
    mats = {"q_proj": rng.standard_normal((nh * hd, d)), "k_proj": rng.standard_normal((nkv * hd, d)),
            "v_proj": rng.standard_normal((nkv * hd, d)), "o_proj": np.zeros((d, nh * hd)),
            "gate_proj": rng.standard_normal((inter, d)), "up_proj": rng.standard_normal((inter, d)),
            "down_proj": np.zeros((d, inter))}
    p = {"ln1": np.ones(d), "ln2": np.ones(d), "q_b": 0.0, "k_b": 0.0, "v_b": 0.0}
    out = layer.layer_forward(h, p, lambda name, x: x @ mats[name].T, nh, nkv)
    assert np.array_equal(out, h)


# ---------------------------------------------------------------- the whole layer, by scalar loops

def _bf16_scalar(v: float) -> float:
    """fp32 rounding of v, then the nearest value with 8 significant bits, ties to even (Python's
    round() on the exactly scaled significand) -- independent of the oracle's bit manipulation."""
    v = struct.unpack("<f", struct.pack("<f", v))[0]
    if v == 0.0:
        return 0.0
    _, ex = math.frexp(v)
    quantum = math.ldexp(1.0, ex - 8)
    return round(v / quantum) * quantum


def _scalar_layer(h, mats, ln1, ln2, bq, bk, bv, nh, nkv, swap_gate_up=False, ln1_for_mlp=False,
                  drop_qkv_bias=False, round_inputs=True):
    """One Qwen2-shaped decoder layer with Python floats and explicit loops (no numpy), with
    switches that plant the wiring mistakes the oracle must not make."""
    t_len, d = len(h), len(h[0])

    def rms(vec, w):
        r = math.sqrt(sum(x * x for x in vec) / len(vec) + layer.RMS_EPS)
        return [vec[i] / r * w[i] for i in range(len(vec))]

    def lin(name, vec):
        x = [_bf16_scalar(v) for v in vec] if round_inputs else list(vec)
        return [sum(row[k] * x[k] for k in range(len(x))) for row in mats[name]]

    hd = len(mats["q_proj"]) // nh
    qs, ks, vs = [], [], []
    for t in range(t_len):
        a = rms(h[t], ln1)
        q, k, v = lin("q_proj", a), lin("k_proj", a), lin("v_proj", a)
        if not drop_qkv_bias:
            q = [q[i] + bq[i] for i in range(len(q))]
            k = [k[i] + bk[i] for i in range(len(k))]
            v = [v[i] + bv[i] for i in range(len(v))]
        qs.append(q), ks.append(k), vs.append(v)
    out = []
    for t in range(t_len):
        att = []
        for head in range(nh):
            kv = head // (nh // nkv)
            logits = [sum(qs[t][head * hd + i] * ks[u][kv * hd + i] for i in range(hd)) / math.sqrt(hd)
                      for u in range(t + 1)]
            mx = max(logits)
            e = [math.exp(l - mx) for l in logits]
            den = sum(e)
            att += [sum(e[u] / den * vs[u][kv * hd + i] for u in range(t + 1)) for i in range(hd)]
        o = lin("o_proj", att)
        h1 = [h[t][i] + o[i] for i in range(d)]
        b = rms(h1, ln1 if ln1_for_mlp else ln2)
        gate, up = lin("gate_proj", b), lin("up_proj", b)
        if swap_gate_up:
            gate, up = up, gate
        act = [gate[i] / (1.0 + math.exp(-gate[i])) * up[i] for i in range(len(gate))]
        dn = lin("down_proj", act)
        out.append([h1[i] + dn[i] for i in range(d)])
    return out


def _layer_case(seed):
    rng = np.random.default_rng(seed)
    d, nh, nkv, hd, inter, t = 16, 4, 2, 4, 24, 3
    shapes = {"q_proj": (nh * hd, d), "k_proj": (nkv * hd, d), "v_proj": (nkv * hd, d), "o_proj": (d, nh * hd),
              "gate_proj": (inter, d), "up_proj": (inter, d), "down_proj": (d, inter)}
    mats = {name: rng.standard_normal(s) * 0.4 for name, s in shapes.items()}
    ln1, ln2 = rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d)
    bq, bk, bv = (rng.standard_normal(n) * 0.5 for n in (nh * hd, nkv * hd, nkv * hd))
    h = rng.standard_normal((t, d)) * 1.3
    return h, mats, ln1, ln2, bq, bk, bv, nh, nkv


def test_layer_forward_matches_scalar_loops():
    """The oracle's decoder layer against an independent scalar-loop layer on a tiny
    grouped-query case (T = 3, four query heads over two K/V heads, distinct gate / up
    matrices, distinct ln1 / ln2 weights, q / k / v biases, bf16-rounded linear inputs)."""
    h, mats, ln1, ln2, bq, bk, bv, nh, nkv = _layer_case(6)
    p = {"ln1": ln1, "ln2": ln2, "q_b": bq, "k_b": bk, "v_b": bv}
    got = layer.layer_forward(h, p, lambda name, x: x @ mats[name].T, nh, nkv)
    want = np.array(_scalar_layer(h.tolist(), {k: v.tolist() for k, v in mats.items()}, ln1.tolist(), ln2.tolist(),
                                  bq.tolist(), bk.tolist(), bv.tolist(), nh, nkv))
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("mistake", ["swap_gate_up", "ln1_for_mlp", "drop_qkv_bias", "round_inputs"])
def test_layer_case_separates_wiring_mistakes(mistake):
    """The scalar-loop case above is discriminating: each planted mistake (gate and up swapped,
    ln1 used before the MLP, q / k / v biases dropped, linear inputs not rounded to bf16)
    moves the output far beyond the comparison's tolerance."""
    h, mats, ln1, ln2, bq, bk, bv, nh, nkv = _layer_case(6)
    args = (h.tolist(), {k: v.tolist() for k, v in mats.items()}, ln1.tolist(), ln2.tolist(), bq.tolist(),
            bk.tolist(), bv.tolist(), nh, nkv)
    good = np.array(_scalar_layer(*args))
    flags = {"round_inputs": False} if mistake == "round_inputs" else {mistake: True}
    bad = np.array(_scalar_layer(*args, **flags))
    assert np.abs(bad - good).max() > 1e-6 * np.abs(good).max()


def test_single_token_layer_closed_form():
    """T = 1: causal attention over one token returns its value row, so the layer is
    h + o(v(a)) + down(silu(gate(b)) * up(b)) with a = rms(h) ln1, b = rms(h1) ln2; written
    out with numpy from those formulas (biases included)."""
    h, mats, ln1, ln2, bq, bk, bv, nh, nkv = _layer_case(7)
    h = h[:1]
    p = {"ln1": ln1, "ln2": ln2, "q_b": bq, "k_b": bk, "v_b": bv}
    got = layer.layer_forward(h, p, lambda name, x: x @ mats[name].T, nh, nkv)
    r = lambda x: np.array([_bf16_scalar(float(v)) for v in x.ravel()]).reshape(x.shape)  # noqa: E731
    a = h / np.sqrt((h * h).mean() + layer.RMS_EPS) * ln1
    v = r(a) @ mats["v_proj"].T + bv
    hd = mats["q_proj"].shape[0] // nh
    att = np.concatenate([v[:, (hh // (nh // nkv)) * hd:(hh // (nh // nkv) + 1) * hd] for hh in range(nh)], axis=1)
    h1 = h + r(att) @ mats["o_proj"].T
    b = h1 / np.sqrt((h1 * h1).mean() + layer.RMS_EPS) * ln2
    g, u = r(b) @ mats["gate_proj"].T, r(b) @ mats["up_proj"].T
    want = h1 + r(g / (1 + np.exp(-g)) * u) @ mats["down_proj"].T
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())
