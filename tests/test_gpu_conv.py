"""Causal conv1d + SiLU pre-pass on the GPU vs the fp64 oracle."""
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn
from gpu_util import DEV, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,width,planes", [(torch.float32, 4, 1), (torch.bfloat16, 4, 3),
                                                (torch.bfloat16, 3, 1), (torch.float32, 2, 2)])
def test_conv_vs_oracle(dtype, width, planes):
    say(f"case conv {dtype} width={width} planes={planes}")
    g = torch.Generator().manual_seed(20)
    lengths = [1, 5, 130, 2, 64]
    T, ch = sum(lengths), 48 * planes
    x = torch.randn(T, ch, generator=g).to(dtype)
    w = torch.randn(ch, width, generator=g) / 2
    cu = torch.tensor([0] + list(torch.cumsum(torch.tensor(lengths), 0)), dtype=torch.int32)
    y = gdn.gdn_conv1d_silu(*to_dev(x, w, cu), planes=planes).cpu()
    torch.cuda.synchronize()
    ref = oracle.conv1d_silu(x, w, cu)
    pc = ch // planes
    got = torch.cat([y[p] for p in range(planes)], dim=1)
    bar = 1e-5 if dtype == torch.float32 else 1e-2
    assert oracle.rel_err(got, ref) <= bar
    assert got.shape == (T, ch) and y.shape == (planes, T, pc)
