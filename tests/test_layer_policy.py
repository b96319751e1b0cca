"""The per-layer 4/8-bit policy: plan resolution and its fail-fast errors (CPU, no kernel is
called), following "模型量化指南" (blog.yoooo.fun), "混合精度（按层 4/8-bit）" and "共同约定"."""
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
