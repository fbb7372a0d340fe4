"""The allocation-free prefill (gdn_prefill_chunked_noalloc) on the GPU, through the C ABI.

Its workspace is the library's per-GPU scratch array instead of a caller-provided buffer;
the kernels are the same. Two calls in a row, the second with a smaller input, must each
reproduce gdn_prefill_chunked bit for bit (outputs and final states) and meet the oracle's
bar; a call beyond the scratch size is rejected before any launch and changes no memory.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, oracle_prefill, say, to_dev

pytestmark = pytest.mark.gpu


def _both(x):
    """(o, pool) from the workspace prefill and from the allocation-free one, same inputs."""
    n, H, dk, dv = x.n_seqs, x.q.shape[1], x.q.shape[2], x.v.shape[2]
    pool0 = x.init_states.clone().float()
    out = []
    for fn in (gdn.gdn_prefill_chunked, gdn.gdn_prefill_chunked_noalloc):
        q, k, v, g, b, cu, pd = to_dev(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool0.clone())
        slots = torch.arange(n, dtype=torch.int32, device=DEV)
        hi = torch.ones(n, dtype=torch.int32, device=DEV)
        o = fn(q, k, v, g, b, cu, x.chunk, pd, slots, has_init=hi, scale=x.scale,
               qk_l2norm=x.qk_l2norm)
        torch.cuda.synchronize()
        out.append((o.cpu(), pd.cpu()))
    return out


@pytest.mark.parametrize("dtype,perkey", [(torch.bfloat16, True), (torch.bfloat16, False),
                                          (torch.float32, True)])
def test_noalloc_prefill_two_calls_match_workspace_prefill(dtype, perkey):
    big = inputs.random_prefill(81, [1500, 700, 1], H=8, dk=128, dv=128, dtype=dtype,
                                perkey=perkey, with_init=True)
    small = inputs.random_prefill(82, [90, 33], H=2, dk=64, dv=64, dtype=dtype,
                                  perkey=perkey, chunk=32, with_init=True)
    for name, x in (("first, larger", big), ("second, smaller", small)):
        say(f"case noalloc prefill {dtype} perkey={perkey}: {name} call")
        (o_ws, p_ws), (o_na, p_na) = _both(x)
        assert torch.equal(o_na, o_ws) and torch.equal(p_na, p_ws)
        o_ref, s_ref = oracle_prefill(x)
        e_o, e_s = oracle.rel_err(o_na, o_ref), oracle.rel_err(p_na, s_ref)
        say(f"   bit-identical to the workspace prefill; vs oracle o={e_o:.2e} S={e_s:.2e}")
        assert np.isfinite(o_na.float().numpy()).all()
        assert e_o <= BAR[dtype] and e_s <= BAR[dtype]


@pytest.mark.parametrize("perkey", [False, True])
def test_noalloc_prefill_wide_then_narrow_tiles(perkey):
    """64 sequences x 4 heads (128-column scan tiles: the scan forms U and, for the scalar
    gate, reads q itself), then a small call (16-column tiles: the prep forms U) over the same
    scratch: each bit-identical to the workspace prefill and within the oracle's bar."""
    lengths = torch.randint(0, 150, (64,), generator=torch.Generator().manual_seed(83)).tolist()
    wide = inputs.random_prefill(84, lengths, H=4, dk=128, dv=128, perkey=perkey,
                                 with_init=True)
    narrow = inputs.random_prefill(85, [200, 7], H=2, dk=128, dv=128, perkey=perkey,
                                   with_init=True)
    for name, x in (("wide tiles", wide), ("then narrow tiles", narrow)):
        say(f"case noalloc prefill bf16 perkey={perkey}: {name}")
        (o_ws, p_ws), (o_na, p_na) = _both(x)
        assert torch.equal(o_na, o_ws) and torch.equal(p_na, p_ws)
        o_ref, s_ref = oracle_prefill(x)
        e_o, e_s = oracle.rel_err(o_na, o_ref), oracle.rel_err(p_na, s_ref)
        say(f"   bit-identical to the workspace prefill; vs oracle o={e_o:.2e} S={e_s:.2e}")
        assert e_o <= BAR[torch.bfloat16] and e_s <= BAR[torch.bfloat16]


@pytest.mark.parametrize("perkey", [False, True])
def test_noalloc_prefill_segmented_scan(perkey):
    """Few (sequence, head) units with long sequences: the scan runs in segments with chain
    and combine passes, their extra workspace sections in the scratch. A 6000-token, 2-head
    call (4 segments), then a 2700-token, 1-head one (2) over the same scratch: each
    bit-identical to the workspace prefill and within the oracle's bar."""
    first = inputs.random_prefill(86, [6000], H=2, dk=128, dv=128, perkey=perkey,
                                  with_init=True)
    second = inputs.random_prefill(87, [2700], H=1, dk=128, dv=128, perkey=perkey,
                                   with_init=True)
    for name, x in (("first, larger", first), ("second, smaller", second)):
        say(f"case noalloc prefill, segmented scan, perkey={perkey}: {name} call")
        (o_ws, p_ws), (o_na, p_na) = _both(x)
        assert torch.equal(o_na, o_ws) and torch.equal(p_na, p_ws)
        o_ref, s_ref = oracle_prefill(x)
        e_o, e_s = oracle.rel_err(o_na, o_ref), oracle.rel_err(p_na, s_ref)
        say(f"   bit-identical to the workspace prefill; vs oracle o={e_o:.2e} S={e_s:.2e}")
        assert e_o <= BAR[torch.bfloat16] and e_s <= BAR[torch.bfloat16]


def test_noalloc_prefill_rejects_oversized_call_without_touching_memory():
    say("case noalloc prefill beyond the scratch size")
    T, H, d = 8192, 16, 128
    need = gdn.gdn_prefill_workspace_bytes(H, d, d, torch.bfloat16, False, 1, T, 64)
    assert need > gdn.GDN_NOALLOC_SCRATCH_BYTES
    x = inputs.prefill_config(0, T=T, H=H, d=d)
    q, k, v, g, b, cu = to_dev(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
    pool = torch.full((1, H, d, d), 7.0, device=DEV)
    o = torch.full((T, H, d), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gdn.GdnError) as err:
        gdn.gdn_prefill_chunked_noalloc(q, k, v, g, b, cu, 64, pool,
                                        torch.zeros(1, dtype=torch.int32, device=DEV),
                                        scale=x.scale, o=o)
    assert err.value.status == 5
    torch.cuda.synchronize()
    assert torch.all(pool == 7.0) and torch.all(o == 3.0)
