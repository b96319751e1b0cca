"""The per-layer 4/8-bit policy: plan resolution and its fail-fast errors, following "模型量化指南"
(blog.yoooo.fun), "混合精度（按层 4/8-bit）" and "共同约定"; and the stacking of one norm's consumers
into one module (W4A16Linear.concat).  CPU only: no kernel is called."""
import pytest
import torch

from weight_only_bit_group_amd.layer import LayerQuantPolicy, W4A16Linear, plan_quantization


class _Block(torch.nn.Module):
    def __init__(self):
        super().__init__()
        self.q_proj = torch.nn.Linear(128, 128, bias=False)
        self.mlp = torch.nn.Module()
        self.mlp.gate_proj = torch.nn.Linear(128, 256, bias=False)
        self.mlp.down_proj = torch.nn.Linear(256, 128, bias=False)


def _model():
    m = torch.nn.Module()
    m.layers = torch.nn.ModuleList([_Block(), _Block()])
    m.lm_head = torch.nn.Linear(128, 64, bias=False)
    return m


def test_policies_override_the_base_and_inherit_the_rest():
    plan = plan_quantization(_model(), ("q_proj", "mlp", "lm_head"), bits=4, group_size=64,
                             layer_policies=(LayerQuantPolicy(("lm_head",), bits=8),
                                             LayerQuantPolicy(("layers.0.mlp",), group_size=128),
                                             LayerQuantPolicy(("layers.0.mlp.down_proj",), sym=True)))
    assert plan["lm_head"] == (8, 64, False)
    assert plan["layers.0.mlp.gate_proj"] == (4, 128, False)
    assert plan["layers.0.mlp.down_proj"] == (4, 128, True)      # later policy wins, group inherited
    assert plan["layers.1.mlp.gate_proj"] == (4, 64, False)
    assert plan["layers.1.q_proj"] == (4, 64, False)
    assert len(plan) == 7


def test_target_matching_is_by_whole_name_components():
    with pytest.raises(ValueError, match="match no linear"):
        plan_quantization(_model(), ("proj",))                     # "proj" is no component
    assert set(plan_quantization(_model(), ("layers.1",))) == {"layers.1.q_proj", "layers.1.mlp.gate_proj",
                                                                 "layers.1.mlp.down_proj"}


def test_fail_fast_errors():
    with pytest.raises(ValueError, match="no torch.nn.Linear"):
        plan_quantization(torch.nn.Sequential(torch.nn.ReLU()), ("q_proj",))
    with pytest.raises(ValueError, match="policy targets"):
        plan_quantization(_model(), ("q_proj",), layer_policies=(LayerQuantPolicy(("lm_head",), bits=8),))
    with pytest.raises(ValueError, match="unsupported"):
        plan_quantization(_model(), ("lm_head",), bits=8, sym=True)
    with pytest.raises(ValueError, match="unsupported"):
        plan_quantization(_model(), ("lm_head",), bits=3)
    with pytest.raises(ValueError, match="multiple of group_size"):
        m = _model()
        m.odd = torch.nn.Linear(96, 8)
        plan_quantization(m, ("odd",), group_size=64)
    m = _model()
    m.lm_head = W4A16Linear(torch.zeros((64, 64), dtype=torch.uint8), torch.zeros((64, 2)),
                            torch.zeros((64, 2), dtype=torch.uint8), 64)
    with pytest.raises(ValueError, match="already quantized"):
        plan_quantization(m, ("lm_head",))


def _packed(n, k, g, bias=None, fill=0):
    """A W4A16Linear over hand-made CPU buffers (no kernel runs: construction and concat only)."""
    return W4A16Linear(torch.full((n, k // 2), fill, dtype=torch.uint8), torch.full((n, k // g), 0.5),
                       torch.full((n, k // g), 3, dtype=torch.uint8), g, bias)


def test_concat_stacks_rows_scales_zeros_and_biases():
    q = _packed(8, 64, 32, bias=torch.arange(8, dtype=torch.float32), fill=1)
    k = _packed(4, 64, 32, fill=2)                      # no bias: zeros in the stacked bias
    v = _packed(4, 64, 32, bias=torch.ones(4), fill=3)
    f = W4A16Linear.concat([q, k, v])
    assert f.split_sizes == [8, 4, 4] and f.out_features == 16 and f.in_features == 64 and f.group == 32
    assert torch.equal(f.packed, torch.cat([q.packed, k.packed, v.packed]))
    assert torch.equal(f.scales, torch.cat([q.scales, k.scales, v.scales]))
    assert torch.equal(f.zeros, torch.cat([q.zeros, k.zeros, v.zeros]))
    assert torch.equal(f.bias, torch.cat([torch.arange(8, dtype=torch.float32), torch.zeros(4), torch.ones(4)]))
    assert W4A16Linear.concat([k, k]).bias is None       # no module has a bias


def test_concat_refuses_mismatched_modules():
    with pytest.raises(ValueError, match="share in_features and group"):
        W4A16Linear.concat([_packed(8, 64, 32), _packed(8, 128, 32)])
    with pytest.raises(ValueError, match="share in_features and group"):
        W4A16Linear.concat([_packed(8, 64, 32), _packed(8, 64, 64)])
    with pytest.raises(TypeError):
        W4A16Linear.concat([_packed(8, 64, 32), torch.nn.Linear(64, 8)])
    with pytest.raises(ValueError):
        W4A16Linear.concat([])


def test_quantized_modules_keep_no_staging_buffer(monkeypatch):
    """The staged GEMM's bf16 staging matrix (N * K * 2 bytes, as large as the dense weight) is a
    per-call allocation: after a forward at M = 2048 the module holds only its packed triple
    (and bias), so swapping linears for W4A16Linear keeps the memory saving.  CPU only: the
    binding's GEMM is replaced by a stand-in that allocates the staging matrix as the binding
    does and returns zeros."""
    from weight_only_bit_group_amd import layer as L
    n, k, g, m = 256, 512, 64, 2048
    seen = []

    def fake_gemm(x, packed, scales, zeros, group, out=None, workspace=None):
        seen.append(workspace)
        staging = torch.empty(n * k * 2, dtype=torch.uint8)   # what the binding allocates per call
        assert staging.numel() == n * k * 2
        return torch.zeros(x.shape[0], packed.shape[0])

    monkeypatch.setattr(L.B, "aq_w4a16_gemm", fake_gemm)
    mod = W4A16Linear(torch.zeros(n, k // 2, dtype=torch.uint8), torch.zeros(n, k // g), torch.zeros(n, k // g,
                      dtype=torch.uint8), g)
    mod(torch.zeros(m, k))
    assert seen == [None]      # no workspace passed in: the binding sizes and frees it per call
    held = sum(t.numel() * t.element_size() for t in list(mod.buffers()) + [v for v in vars(mod).values()
                                                                              if isinstance(v, torch.Tensor)])
    assert held == n * k // 2 + n * (k // g) * 5
    assert not any(isinstance(v, torch.Tensor) and v.numel() * v.element_size() >= n * k * 2
                   for v in vars(mod).values())
