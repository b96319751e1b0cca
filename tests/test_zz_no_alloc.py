"""The allocation-free abs-mean entry point (aq_act_absmean_noalloc, the library's own
device scratch) against aq_act_absmean with a caller workspace: bit-identical sums and
means on two calls in a row, the second smaller, and accumulation across them."""
import numpy as np
import pytest
import torch

from tests.gpu_util import host, step
from weight_only_bit_group_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _x(seed, t, k):
    bits = synth.calibration_rows_bf16(seed, t, k)
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def test_noalloc_absmean_equals_workspace_entry():
    from weight_only_bit_group_amd import binding as B
    dev = torch.device("cuda")
    # the larger call first (most of the scratch written), then a smaller, ragged one: the
    # second must not see the first call's partials
    for t, k in ((16384, 2048), (1000, 136)):
        step(f"aq_act_absmean_noalloc T={t} K={k}")
        x = _x(7 + k, t, k)
        s_ref = torch.zeros(k, dtype=torch.float64, device=dev)
        m_ref = torch.empty(k, dtype=torch.float32, device=dev)
        B.aq_act_absmean(x, s_ref, t, m_ref)
        s_na = torch.zeros(k, dtype=torch.float64, device=dev)
        m_na = torch.empty(k, dtype=torch.float32, device=dev)
        B.aq_act_absmean_noalloc(x, s_na, t, m_na)
        assert np.array_equal(host(s_na).view(np.uint64), host(s_ref).view(np.uint64))
        assert np.array_equal(host(m_na).view(np.uint32), host(m_ref).view(np.uint32))
    # two chunks accumulated into one sum: the same as the workspace entry point's two calls
    step("aq_act_absmean_noalloc, two accumulated chunks")
    k = 512
    xa, xb = _x(21, 3000, k), _x(22, 700, k)
    s_ref = torch.zeros(k, dtype=torch.float64, device=dev)
    m_ref = torch.empty(k, dtype=torch.float32, device=dev)
    B.aq_act_absmean(xa, s_ref, 3000)
    B.aq_act_absmean(xb, s_ref, 3700, m_ref)
    s_na = torch.zeros(k, dtype=torch.float64, device=dev)
    m_na = torch.empty(k, dtype=torch.float32, device=dev)
    B.aq_act_absmean_noalloc(xa, s_na, 3000)
    B.aq_act_absmean_noalloc(xb, s_na, 3700, m_na)
    assert np.array_equal(host(s_na).view(np.uint64), host(s_ref).view(np.uint64))
    assert np.array_equal(host(m_na).view(np.uint32), host(m_ref).view(np.uint32))
