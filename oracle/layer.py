"""Norm-group AWQ, the RMSNorm fold and a quantized decoder layer's forward.

Test infrastructure only (see the package docstring).

Sources
  * "Lance-Quant" page (zingnex.cn), section "量化应用：网格搜索与分组策略":
    awq_apply grid-searches the AWQ scale for each normalisation together with
    the linears that consume its output, folds the scale into the preceding
    RMSNorm and packs the weights group-wise to INT4.
  * Same page, the paragraph after the fourth case: o_proj and down_proj
    follow a non-linearity, so no scale can be folded into a norm before them;
    they get plain group-wise quantization.
  * Same page, "运行时替换与内存优化": the linears of the model are replaced by
    quantized linear modules for inference.
  * "模型量化指南" (blog.yoooo.fun), "共同约定": the quantized layer dequantizes
    in memory and is mathematically the original layer with W replaced by its
    dequantized value.
  * The equivalent transform (X / s)(s W) = X W, OmniQuant tutorial (cyqw.cn),
    section 2.2.2.

Readings (listed in the design notes)
  * A joint search over the consumers of one norm is the single-matrix search
    on their weights concatenated along N (rows); the output MSE is then the
    mean over T x (N_1 + N_2 + ...) elements.
  * The fold divides the fp32 norm weight by the chosen scale: w' = fl32(w / s).
  * The decoder layer is the Qwen2 shape: RMSNorm (eps 1e-6) -> q, k, v (with
    bias) -> causal grouped-query softmax attention -> o (no bias) ->
    residual; RMSNorm -> gate, up -> SiLU(gate) * up -> down -> residual.  The
    positional rotation is left out: it acts between the projections and the
    softmax and touches no quantized weight.
  * Every linear receives its input rounded to bf16 (round half to even), as
    the W4A16 kernels take bf16 activations; everything else is fp64.
"""
from __future__ import annotations

import numpy as np

from . import awq, int4, stats

RMS_EPS = 1e-6


def bf16_round(a) -> np.ndarray:
    """fp32 -> bf16 -> fp32 with round half to even (finite inputs)."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def rms_norm(h, w, eps: float = RMS_EPS) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * w over the last axis, fp64."""
    h = np.asarray(h, dtype=np.float64)
    r = np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h / r * np.asarray(w, dtype=np.float64)


def silu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def causal_attention(q, k, v, n_heads: int, n_kv: int) -> np.ndarray:
    """Softmax attention over the token axis with a causal mask, grouped K/V heads, fp64."""
    t = q.shape[0]
    hd = q.shape[1] // n_heads
    out = np.zeros_like(q, dtype=np.float64)
    mask = np.triu(np.ones((t, t), dtype=bool), 1)
    for h in range(n_heads):
        kv = h // (n_heads // n_kv)
        qh = q[:, h * hd:(h + 1) * hd]
        kh = k[:, kv * hd:(kv + 1) * hd]
        vh = v[:, kv * hd:(kv + 1) * hd]
        a = qh @ kh.T / np.sqrt(hd)
        a[mask] = -np.inf
        a = np.exp(a - a.max(axis=1, keepdims=True))
        a /= a.sum(axis=1, keepdims=True)
        out[:, h * hd:(h + 1) * hd] = a @ vh
    return out


def norm_group_awq(x_norm, norm_w, weights, group: int, n_grid: int = 20, search_tokens: int = 4096):
    """AWQ for one norm and its consumers.

    x_norm: the norm's output over the calibration tokens [T, K] (fp32 values);
    weights: list of [N_i, K] matrices consuming it.  Returns dict(norm = folded
    fp32 norm weight, packs = [(packed, scales, zeros)] per matrix, search = the
    search result on the concatenated weights).
    """
    x = np.asarray(x_norm, dtype=np.float32)
    mean = stats.absmean(x)
    w_cat = np.concatenate([np.asarray(w, dtype=np.float32) for w in weights], axis=0)
    res = awq.search(x[:search_tokens], mean, w_cat, group, n_grid)
    folded = (np.asarray(norm_w, dtype=np.float32) / res["scale"]).astype(np.float32)
    packs, n0 = [], 0
    for w in weights:
        n1 = n0 + w.shape[0]
        packs.append((res["packed"][n0:n1], res["scales"][n0:n1], res["zeros"][n0:n1]))
        n0 = n1
    return {"norm": folded, "packs": packs, "search": res}


def layer_forward(h, p, linear, n_heads: int, n_kv: int) -> np.ndarray:
    """One decoder layer on hidden states h [T, D], fp64.

    p: dict with "ln1", "ln2" (norm weights) and the biases "q_b", "k_b", "v_b";
    linear(name, x) returns x @ W_name^T for an fp64 input x [T, K].
    """
    h = np.asarray(h, dtype=np.float64)
    lin = lambda name, x: linear(name, bf16_round(x).astype(np.float64))  # noqa: E731
    a = rms_norm(h, p["ln1"])
    q = lin("q_proj", a) + p["q_b"]
    k = lin("k_proj", a) + p["k_b"]
    v = lin("v_proj", a) + p["v_b"]
    h = h + lin("o_proj", causal_attention(q, k, v, n_heads, n_kv))
    b = rms_norm(h, p["ln2"])
    return h + lin("down_proj", silu(lin("gate_proj", b)) * lin("up_proj", b))


def dequantized_linear(packs: dict, group: int):
    """linear(name, x) = x @ dequantize(packs[name])^T in fp64."""
    mats = {name: int4.dequantize(pk, sc, zr, group) for name, (pk, sc, zr) in packs.items()}
    return lambda name, x: x @ mats[name].T
