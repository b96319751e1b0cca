"""GPU parity of the module-level path: norm-group AWQ with the RMSNorm fold, plain packing of
o_proj / down_proj, and a decoder layer whose linears are swapped for W4A16Linear, against the
oracle (oracle/layer.py) on the same calibration bytes."""
import numpy as np
import pytest
import torch

from oracle import int4, layer
from tests.gpu_util import check_close, host, step
from weight_only_bit_group_amd import synth

pytestmark = pytest.mark.gpu

D, NH, NKV, HD, INTER, G = 512, 4, 2, 128, 1408, 64
T_CAL, T_TEST = 512, 24


@pytest.fixture(scope="module", autouse=True)
def _gpu(lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_only_bit_group_amd import layer as L
    globals()["L"] = L


def _weights(seed):
    rng = np.random.default_rng(seed)
    shapes = {"q_proj": (NH * HD, D), "k_proj": (NKV * HD, D), "v_proj": (NKV * HD, D), "o_proj": (D, NH * HD),
              "gate_proj": (INTER, D), "up_proj": (INTER, D), "down_proj": (D, INTER)}
    w = {n: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(synth.weight_f32(rng, *s, 0.02, outlier_frac=0.001)))
         for n, s in shapes.items()}
    p = {"ln1": rng.uniform(0.8, 1.2, D).astype(np.float32), "ln2": rng.uniform(0.8, 1.2, D).astype(np.float32),
         "q_b": (rng.standard_normal(NH * HD) * 0.1).astype(np.float32),
         "k_b": (rng.standard_normal(NKV * HD) * 0.1).astype(np.float32),
         "v_b": (rng.standard_normal(NKV * HD) * 0.1).astype(np.float32)}
    return w, p


def _torch_layer(h, p, linear):
    """The decoder layer in torch fp32 (the same structure as the oracle's)."""
    def rms(x, w):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + layer.RMS_EPS) * w

    t = h.shape[0]
    a = rms(h, p["ln1"])
    q, k, v = linear("q_proj", a), linear("k_proj", a), linear("v_proj", a)
    qh = q.view(t, NH, HD).transpose(0, 1)
    kh = k.view(t, NKV, HD).transpose(0, 1).repeat_interleave(NH // NKV, 0)
    vh = v.view(t, NKV, HD).transpose(0, 1).repeat_interleave(NH // NKV, 0)
    s = qh @ kh.transpose(1, 2).contiguous() / HD ** 0.5
    s = s.masked_fill(torch.triu(torch.ones(t, t, dtype=torch.bool, device=h.device), 1), float("-inf"))
    att = (torch.softmax(s, -1) @ vh).transpose(0, 1).reshape(t, NH * HD)
    h = h + linear("o_proj", att)
    b = rms(h, p["ln2"])
    return h + linear("down_proj", torch.nn.functional.silu(linear("gate_proj", b)) * linear("up_proj", b))


def test_decoder_layer_norm_group_awq_and_module_swap():
    w, p = _weights(11)
    dev = torch.device("cuda")
    rng = np.random.default_rng(12)
    h_cal = torch.from_numpy(synth.activations_f32(rng, T_CAL, D, round(0.01 * D))).to(dev)
    h_test = torch.from_numpy(synth.activations_f32(rng, T_TEST, D, round(0.01 * D))).to(dev)
    pt = {k: torch.from_numpy(v).to(dev) for k, v in p.items()}
    lin = {n: torch.nn.Linear(m.shape[1], m.shape[0], bias=n in ("q_proj", "k_proj", "v_proj")).to(dev)
           for n, m in w.items()}
    with torch.no_grad():
        for n, m in w.items():
            lin[n].weight.copy_(torch.from_numpy(m))
            if lin[n].bias is not None:
                lin[n].bias.copy_(pt[n[0] + "_b"])

    # calibration pass through the original layer: capture the two norm outputs (bf16)
    cap = {}

    def orig(name, x):
        if name in ("q_proj", "gate_proj"):
            cap[name] = x.to(torch.bfloat16).contiguous()
        return torch.nn.functional.linear(x.to(torch.bfloat16).float(), lin[name].weight, lin[name].bias)

    step("calibration pass (torch) on the original layer")
    with torch.no_grad():
        _torch_layer(h_cal, pt, orig)
    step("norm_group_awq q|k|v and gate|up, plain o / down")
    ln1, (q, k, v), r1 = L.norm_group_awq(pt["ln1"], [lin["q_proj"], lin["k_proj"], lin["v_proj"]], cap["q_proj"],
                                          G, 20, T_CAL)
    ln2, (gt, up), r2 = L.norm_group_awq(pt["ln2"], [lin["gate_proj"], lin["up_proj"]], cap["gate_proj"], G, 20,
                                         T_CAL)
    mods = {"q_proj": q, "k_proj": k, "v_proj": v, "gate_proj": gt, "up_proj": up,
            "o_proj": L.quantize_linear(lin["o_proj"], G), "down_proj": L.quantize_linear(lin["down_proj"], G)}
    with pytest.raises(ValueError):
        L.quantize_linear(mods["o_proj"], G)   # already quantized

    # oracle on the same calibration bytes
    x1 = synth.bf16_bits_to_f32(host(cap["q_proj"].view(torch.int16)).view(np.uint16))
    x2 = synth.bf16_bits_to_f32(host(cap["gate_proj"].view(torch.int16)).view(np.uint16))
    o1 = layer.norm_group_awq(x1, p["ln1"], [w["q_proj"], w["k_proj"], w["v_proj"]], G, 20, T_CAL)
    o2 = layer.norm_group_awq(x2, p["ln2"], [w["gate_proj"], w["up_proj"]], G, 20, T_CAL)
    for r, o, what in ((r1, o1, "q|k|v"), (r2, o2, "gate|up")):
        print(f"[gpu] {what}: best alpha index gpu {int(host(r['best'])[0])} oracle {o['search']['best']}",
              flush=True)
        assert int(host(r["best"])[0]) == o["search"]["best"]
        assert np.array_equal(host(r["best_scale"]).view(np.uint32), o["search"]["scale"].view(np.uint32))
    assert np.array_equal(host(ln1).view(np.uint32), o1["norm"].view(np.uint32))
    assert np.array_equal(host(ln2).view(np.uint32), o2["norm"].view(np.uint32))
    packs = {}
    for names, o in ((("q_proj", "k_proj", "v_proj"), o1), (("gate_proj", "up_proj"), o2)):
        for n, trip in zip(names, o["packs"]):
            packs[n] = trip
    packs["o_proj"] = int4.quantize_pack(w["o_proj"], G)
    packs["down_proj"] = int4.quantize_pack(w["down_proj"], G)
    for n, (pk, sc, zr) in packs.items():
        m = mods[n]
        assert np.array_equal(host(m.packed), pk) and np.array_equal(host(m.scales).view(np.uint32),
                                                                   sc.view(np.uint32)) \
            and np.array_equal(host(m.zeros), zr), n

    # the consumers of each norm fused into one module: every slice of its output equals the
    # separate module's output (rows are independent), at the GEMV and GEMM sizes
    for names in (("q_proj", "k_proj", "v_proj"), ("gate_proj", "up_proj")):
        fused = L.W4A16Linear.concat([mods[n] for n in names])
        assert fused.split_sizes == [mods[n].out_features for n in names]
        for rows in (1, T_TEST):
            step(f"fused {'|'.join(names)} forward, {rows} token(s)")
            with torch.no_grad():
                x = cap[names[0]][:rows].float()
                parts = torch.split(fused(x), fused.split_sizes, -1)
                for n, part in zip(names, parts):
                    assert torch.equal(part, mods[n](x)), (n, rows)
    with pytest.raises(ValueError):
        L.W4A16Linear.concat([mods["q_proj"], mods["down_proj"]])   # different in_features

    # forward of the quantized layer (GEMM at T_TEST rows, GEMV at one row) against the oracle
    pq = dict(pt, ln1=ln1, ln2=ln2)
    po = dict(p, ln1=o1["norm"], ln2=o2["norm"])
    for rows in (T_TEST, 1):
        step(f"quantized decoder layer forward, {rows} token(s)")
        with torch.no_grad():
            y = host(_torch_layer(h_test[:rows], pq, lambda n, x: mods[n](x)))
        ref = layer.layer_forward(host(h_test[:rows]), po, layer.dequantized_linear(packs, G), NH, NKV)
        hx = host(h_test[:rows]).astype(np.float64)
        check_close(y - hx, ref - hx, f"decoder layer branch sum, {rows} token(s)")
        check_close(y, ref, f"decoder layer output, {rows} token(s)")


def test_quantize_modules_mixed_4_8_bit_policy():
    """quantize_modules swaps the selected linears following the policies (lm_head at 8 bits, one
    block's MLP at g=128 symmetric, the rest 4-bit g=64); each swapped module's output equals the
    oracle's packing + fp64 forward of the same weight within the tolerance."""
    torch.manual_seed(0)
    dev_ = torch.device("cuda")
    model = torch.nn.Module()
    model.layers = torch.nn.ModuleList()
    for _ in range(2):
        blk = torch.nn.Module()
        blk.q_proj = torch.nn.Linear(512, 512, bias=True)
        blk.mlp = torch.nn.Module()
        blk.mlp.down_proj = torch.nn.Linear(1408, 512, bias=False)
        model.layers.append(blk)
    model.lm_head = torch.nn.Linear(512, 1024, bias=False)
    model = model.to(dev_)
    weights = {n: m.weight.detach().float().cpu().numpy() for n, m in model.named_modules()
               if isinstance(m, torch.nn.Linear)}
    biases = {n: (m.bias.detach().float().cpu().numpy() if m.bias is not None else 0.0)
              for n, m in model.named_modules() if isinstance(m, torch.nn.Linear)}
    step("quantize_modules with a 4/8-bit policy")
    plan = L.quantize_modules(model, ("q_proj", "mlp", "lm_head"), bits=4, group_size=64,
                              layer_policies=(L.LayerQuantPolicy(("lm_head",), bits=8),
                                              L.LayerQuantPolicy(("layers.1.mlp",), group_size=128, sym=True)))
    assert plan["lm_head"] == (8, 64, False) and plan["layers.1.mlp.down_proj"] == (4, 128, True)
    named = dict(model.named_modules())
    assert isinstance(named["lm_head"], L.W8A16Linear) and isinstance(named["layers.0.q_proj"], L.W4A16Linear)
    for name, (bits, g, sym) in plan.items():
        k = weights[name].shape[1]
        for m in (1, 40):
            xb = synth.layer_activations_bf16(9, m, k)
            x = synth.bf16_bits_to_f32(xb)
            step(f"{name} bits={bits} g={g} sym={sym} M={m}")
            y = host(named[name](torch.from_numpy(x).to(dev_)))
            if bits == 8:
                ref = int4.forward8(x, *int4.quantize_codes8(weights[name], g), g)
            else:
                trip = int4.quantize_pack_sym(weights[name], g) if sym else int4.quantize_pack(weights[name], g)
                ref = int4.forward(x, *trip, g)
            check_close(y, ref + biases[name], f"policy {name} M={m}")


def test_fold_norm_is_the_ieee_quotient():
    """aq_awq_fold_norm: fl32(w / s) per channel, bit for bit, for fp32 and bf16 norm weights
    (bf16 widened exactly), with scales spanning many binades and a ragged K."""
    from weight_only_bit_group_amd import binding as B
    rng = np.random.default_rng(12)
    k = 2049
    w = rng.uniform(0.5, 1.5, k).astype(np.float32)
    s = np.exp(rng.uniform(-8, 8, k)).astype(np.float32)
    step("aq_awq_fold_norm fp32 / bf16, K = 2049")
    got = host(B.aq_awq_fold_norm(torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda()))
    assert np.array_equal(got.view(np.uint32), (w / s).astype(np.float32).view(np.uint32))
    wb = synth.f32_to_bf16_bits(w)
    got = host(B.aq_awq_fold_norm(torch.from_numpy(wb.view(np.int16)).cuda().view(torch.bfloat16),
                                  torch.from_numpy(s).cuda()))
    want = (synth.bf16_bits_to_f32(wb) / s).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
