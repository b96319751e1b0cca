"""Quantized linear module and the norm-group AWQ apply step, on top of the binding.

Every computation is a libaq call (pack, abs-mean, alpha search, GEMV / GEMM);
this module only arranges tensors and swaps modules.

  * ``W4A16Linear``: the drop-in replacement of an ``nn.Linear`` holding the
    packed INT4 triple; its forward is the W4A16 GEMV (M <= 16 rows) or GEMM
    ("Lance-Quant", zingnex.cn, "运行时替换与内存优化": linears replaced by
    quantized linear modules; "模型量化指南", blog.yoooo.fun, "共同约定": the
    quantized layer dequantizes in memory and equals the original layer with W
    replaced by its dequantized value, and quantizing an already quantized
    layer is refused).
  * ``norm_group_awq``: AWQ for one normalisation and the linears consuming its
    output ("Lance-Quant", "量化应用：网格搜索与分组策略": grid search of the
    scale per norm and its consumers, the scale folded into the preceding
    RMSNorm, group-wise INT4 packing).  The consumers are searched jointly:
    their weights concatenated along N share one channel scale s, the norm
    weight becomes w / s and each linear holds Q(W diag(s)).
  * ``quantize_linear``: plain group-wise min-max packing for linears with no
    norm in front of them (o_proj and down_proj follow a non-linearity, so no
    scale can be folded; same page, after the fourth case).
  * ``W8A16Linear`` and ``quantize_modules`` with ``LayerQuantPolicy``: the mixed
    4/8-bit policy ("模型量化指南", "混合精度（按层 4/8-bit）": a policy binds bits /
    group size / symmetry to named layers, unspecified fields inherit the base
    configuration, and a policy target outside the layers selected by
    target_modules is an error at parse time; "共同约定": explicit errors for a
    model without linears, targets that match nothing, and re-quantization).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


class W4A16Linear(torch.nn.Module):
    """y = x W^T (+ bias) with W stored as group-wise INT4 (packed [N, K/2], S, z).

    The input is cast to bf16 (the kernels' activation type); the output is fp32.
    """

    def __init__(self, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, group: int,
                 bias: torch.Tensor | None = None):
        super().__init__()
        if packed.dim() != 2 or scales.shape != zeros.shape or scales.shape[0] != packed.shape[0]:
            raise ValueError("packed [N, K/2], scales and zeros [N, K/group] expected")
        self.group = int(group)
        self.in_features = packed.shape[1] * 2
        self.out_features = packed.shape[0]
        if scales.shape[1] * self.group != self.in_features:
            raise ValueError("scales must be [N, K/group]")
        self.register_buffer("packed", packed.contiguous())
        self.register_buffer("scales", scales.contiguous())
        self.register_buffer("zeros", zeros.contiguous())
        self.register_buffer("bias", None if bias is None else bias.detach().float().contiguous())
        self.split_sizes = [self.out_features]

    @classmethod
    def from_weight(cls, weight: torch.Tensor, group: int, chan_scale: torch.Tensor | None = None,
                    bias: torch.Tensor | None = None, sym: bool = False) -> "W4A16Linear":
        """Pack W [N, K] (fp32 or bf16, on the GPU), optionally scaled by chan_scale [K];
        sym=True packs the symmetric variant (same format, zero point 8)."""
        p, s, z = B.aq_quantize_pack(weight.detach().contiguous(), group, chan_scale, sym=sym)
        return cls(p, s, z, group, bias)

    @classmethod
    def concat(cls, mods) -> "W4A16Linear":
        """One module over the stacked output rows of several W4A16Linear with the same input
        size and group (the consumers of one norm, e.g. q|k|v or gate|up): one GEMV / GEMM
        launch instead of one per module.  Output rows are computed independently, so each
        slice of the result equals the separate module's output; ``split_sizes`` gives the
        slice widths (``torch.split(y, m.split_sizes, -1)``)."""
        mods = list(mods)
        if not mods:
            raise ValueError("nothing to concatenate")
        k, g = mods[0].in_features, mods[0].group
        for m in mods:
            if not isinstance(m, W4A16Linear):
                raise TypeError(f"expected W4A16Linear, got {type(m).__name__}")
            if m.in_features != k or m.group != g:
                raise ValueError("modules must share in_features and group")
        bias = None
        if any(m.bias is not None for m in mods):
            bias = torch.cat([m.bias if m.bias is not None else
                              torch.zeros(m.out_features, dtype=torch.float32, device=m.packed.device) for m in mods])
        out = cls(torch.cat([m.packed for m in mods]), torch.cat([m.scales for m in mods]),
                  torch.cat([m.zeros for m in mods]), g, bias)
        out.split_sizes = [m.out_features for m in mods]
        return out

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected {self.in_features} input features, got {x.shape[-1]}")
        x2 = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        m = x2.shape[0]
        if m <= 16:
            y = B.aq_w4a16_gemv(x2, self.packed, self.scales, self.zeros, self.group)
        else:
            # the staging matrix (as large as a bf16 copy of W) is allocated per call: torch's
            # caching allocator hands the block back in stream order, and no module keeps one
            y = B.aq_w4a16_gemm(x2, self.packed, self.scales, self.zeros, self.group)
        if self.bias is not None:
            y = y + self.bias
        return y.reshape(*x.shape[:-1], self.out_features)

    def extra_repr(self) -> str:
        return f"in_features={self.in_features}, out_features={self.out_features}, group={self.group}"


def _weight_of(linear) -> torch.Tensor:
    if isinstance(linear, W4A16Linear):
        raise ValueError("layer is already quantized")
    if not isinstance(linear, torch.nn.Linear):
        raise TypeError(f"expected torch.nn.Linear, got {type(linear).__name__}")
    return linear.weight.detach()


def quantize_linear(linear: torch.nn.Linear, group: int, sym: bool = False) -> W4A16Linear:
    """Plain group-wise INT4 of one linear (no channel scale): min-max asymmetric, or
    symmetric (max |w| / 7, zero point 8) with sym=True."""
    w = _weight_of(linear)
    return W4A16Linear.from_weight(w.contiguous(), group, None, linear.bias, sym)


def norm_group_awq(norm_weight: torch.Tensor, linears, x_norm: torch.Tensor, group: int, n_grid: int = 20,
                   search_tokens: int = 4096):
    """AWQ of the linears consuming one RMSNorm's output.

    x_norm: that norm's output over the calibration tokens [T, K] bf16 (all T
    tokens give the abs-mean statistic; the first ``search_tokens`` score the
    search).  Returns (folded fp32 norm weight [K], [W4A16Linear per linear],
    search dict of aq_awq_search).
    """
    ws = [_weight_of(l) for l in linears]
    if not ws:
        raise ValueError("no linear to quantize")
    k = ws[0].shape[1]
    if any(w.shape[1] != k for w in ws) or any(w.dtype != ws[0].dtype for w in ws):
        raise ValueError("the consumers of one norm must share K and the weight dtype")
    if x_norm.dim() != 2 or x_norm.shape[1] != k:
        raise ValueError(f"x_norm must be [T, {k}]")
    t = x_norm.shape[0]
    x = x_norm.to(torch.bfloat16).contiguous()
    sum_abs = torch.zeros(k, dtype=torch.float64, device=x.device)
    mean = torch.empty(k, dtype=torch.float32, device=x.device)
    B.aq_act_absmean(x, sum_abs, t, mean)          # EINVAL (ValueError) for T == 0
    w_cat = torch.cat(ws, dim=0).contiguous()
    res = B.aq_awq_search(x[:search_tokens].contiguous(), mean.cpu(), w_cat, group, n_grid)
    folded = B.aq_awq_fold_norm(norm_weight.detach().contiguous(), res["best_scale"])
    out, n0 = [], 0
    for lin, w in zip(linears, ws):
        n1 = n0 + w.shape[0]
        out.append(W4A16Linear(res["packed"][n0:n1], res["scales"][n0:n1], res["zeros"][n0:n1], group, lin.bias))
        n0 = n1
    return folded, out, res


class W8A16Linear(torch.nn.Module):
    """y = x W^T (+ bias) with W stored as group-wise INT8 (codes [N, K], S, z); bf16 in, fp32 out."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, group: int,
                 bias: torch.Tensor | None = None):
        super().__init__()
        if codes.dim() != 2 or scales.shape != zeros.shape or scales.shape[0] != codes.shape[0]:
            raise ValueError("codes [N, K], scales and zeros [N, K/group] expected")
        self.group = int(group)
        self.in_features = codes.shape[1]
        self.out_features = codes.shape[0]
        if scales.shape[1] * self.group != self.in_features:
            raise ValueError("scales must be [N, K/group]")
        self.register_buffer("codes", codes.contiguous())
        self.register_buffer("scales", scales.contiguous())
        self.register_buffer("zeros", zeros.contiguous())
        self.register_buffer("bias", None if bias is None else bias.detach().float().contiguous())

    @classmethod
    def from_weight(cls, weight: torch.Tensor, group: int, chan_scale: torch.Tensor | None = None,
                    bias: torch.Tensor | None = None) -> "W8A16Linear":
        c, s, z = B.aq_quantize_pack8(weight.detach().contiguous(), group, chan_scale)
        return cls(c, s, z, group, bias)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected {self.in_features} input features, got {x.shape[-1]}")
        x2 = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        m = x2.shape[0]
        if m <= 16:
            y = B.aq_w8a16_gemv(x2, self.codes, self.scales, self.zeros, self.group)
        else:
            # per-call staging matrix, as for W4A16Linear
            y = B.aq_w8a16_gemm(x2, self.codes, self.scales, self.zeros, self.group)
        if self.bias is not None:
            y = y + self.bias
        return y.reshape(*x.shape[:-1], self.out_features)

    def extra_repr(self) -> str:
        return f"in_features={self.in_features}, out_features={self.out_features}, group={self.group}, bits=8"


@dataclass(frozen=True)
class LayerQuantPolicy:
    """Per-layer override of the base configuration; None fields inherit it."""
    target_modules: tuple
    bits: int | None = None
    group_size: int | None = None
    sym: bool | None = None


def _matches(name: str, target: str) -> bool:
    """target names whole dotted components of name (a linear or one of its parents)."""
    return ("." + target + ".") in ("." + name + ".")


def plan_quantization(model: torch.nn.Module, target_modules, bits: int = 4, group_size: int = 64,
                      sym: bool = False, layer_policies=()):
    """{linear name: (bits, group_size, sym)} for the linears the call would quantize.

    Checks everything before anything is quantized: the model has linears, the
    targets match some, no target is already quantized, every policy target matches
    a selected linear, and every (bits, sym) pair is supported (4-bit asymmetric or
    symmetric, 8-bit asymmetric).
    """
    named = dict(model.named_modules())
    quantized = [n for n, m in named.items() if isinstance(m, (W4A16Linear, W8A16Linear))]
    linears = [n for n, m in named.items() if isinstance(m, torch.nn.Linear)]
    if not linears and not quantized:
        raise ValueError("the model contains no torch.nn.Linear")
    targets = tuple(target_modules)
    hit = [n for n in linears if any(_matches(n, t) for t in targets)]
    again = [n for n in quantized if any(_matches(n, t) for t in targets)]
    if again:
        raise ValueError(f"already quantized: {again[0]}")
    if not hit:
        raise ValueError(f"target_modules {targets} match no linear")
    plan = {n: (bits, group_size, sym) for n in hit}
    for pol in layer_policies:
        sel = [n for n in hit if any(_matches(n, t) for t in pol.target_modules)]
        if not sel:
            raise ValueError(f"policy targets {tuple(pol.target_modules)} match no selected linear")
        for n in sel:
            b, g, s = plan[n]
            plan[n] = (pol.bits if pol.bits is not None else b, pol.group_size if pol.group_size is not None else g,
                       pol.sym if pol.sym is not None else s)
    for n, (b, g, s) in plan.items():
        if b not in (4, 8) or (b == 8 and s) or g not in (32, 64, 128):
            raise ValueError(f"{n}: unsupported configuration bits={b} group_size={g} sym={s}")
        k = named[n].in_features
        if k % g:
            raise ValueError(f"{n}: in_features {k} is not a multiple of group_size {g}")
    return plan


def quantize_modules(model: torch.nn.Module, target_modules, bits: int = 4, group_size: int = 64, sym: bool = False,
                     layer_policies=()):
    """Replace the selected nn.Linear modules of ``model`` by W4A16Linear / W8A16Linear
    (plain group-wise packing) following the base configuration and the policies (the
    last matching policy wins).  Returns the plan of ``plan_quantization``."""
    plan = plan_quantization(model, target_modules, bits, group_size, sym, layer_policies)
    named = dict(model.named_modules())
    for name, (b, g, s) in plan.items():
        lin = named[name]
        new = (W8A16Linear.from_weight(_weight_of(lin).contiguous(), g, None, lin.bias) if b == 8
               else W4A16Linear.from_weight(_weight_of(lin).contiguous(), g, None, lin.bias, s))
        parent_name, _, attr = name.rpartition(".")
        setattr(named[parent_name] if parent_name else model, attr, new)
    return plan
