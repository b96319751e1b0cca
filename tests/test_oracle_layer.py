"""Pins of the norm-group AWQ / fold / decoder-layer oracle (oracle/layer.py)."""
import numpy as np

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
