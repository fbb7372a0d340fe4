"""Prefill with many (sequence, head) units on the GPU vs the fp64 oracle, through the C ABI.

With enough units the scan gives each workgroup 32 to 128 value columns, and then it forms
U = diag(beta) V + ((R - I) diag(beta)) V itself from v (staged through LDS as V^T), with
(R - I) diag(beta) and beta from the prep; for the scalar gate with q given it also reads q
itself and scales each output row by s e^{G_i} / |q_i| instead of reading Q_in. These cases
cover those paths across element types, head dims, chunk sizes (one, two and four 16-token
blocks per chunk), both gates, the in-kernel L2 norm, checkpoints and the fused convolution.
Bars as the other prefill tests: max|x - ref| / max|ref| <= 1e-4 (fp32), 1e-2 (bf16).
"""
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import inputs
from gpu_util import BAR, oracle_prefill, run_prefill, say
from test_gpu_checkpoint import expected_stored, oracle_prefix_states, run_ckpt
from test_gpu_conv_prefill import oracle_conv_prefill, run_fused

pytestmark = pytest.mark.gpu


def tile_width(dtype, units, d):
    """The scan's value-tile width (in 16-column tiles) for a call with `units` (sequence,
    head) pairs: the widest that still leaves one workgroup per CU, at most 4 for fp32."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    tiles, nvb = units * (d // 16), 1
    while nvb * 2 <= d // 16 and tiles // (nvb * 2) >= ncu:
        nvb *= 2
    return min(nvb, 8 if dtype == torch.bfloat16 else 4)


def _lengths(seed, n, hi):
    return torch.randint(0, hi, (n,), generator=torch.Generator().manual_seed(seed)).tolist()


CASES = [
    # (dtype, d, chunk, perkey, n_seqs, H, l2norm in the kernel, initial states)
    (torch.bfloat16, 128, 64, False, 64, 4, True, True),
    (torch.bfloat16, 128, 16, False, 40, 4, False, True),
    (torch.bfloat16, 128, 64, True, 64, 4, True, False),
    (torch.bfloat16, 64, 64, False, 33, 4, True, False),
    (torch.bfloat16, 32, 32, True, 64, 4, False, True),
    (torch.float32, 64, 16, False, 64, 4, True, True),
    (torch.float32, 128, 64, True, 40, 4, False, True),
]


@pytest.mark.parametrize("dtype,d,chunk,perkey,nseq,H,l2,init", CASES)
def test_wide_tiles_vs_oracle(dtype, d, chunk, perkey, nseq, H, l2, init):
    lengths = _lengths(81, nseq, 150)
    lengths[0] = 0
    nvb = tile_width(dtype, nseq * H, d)
    say(f"case wide tiles {dtype} d={d} C={chunk} perkey={perkey} {nseq}x{H} l2={l2} "
        f"init={init}: {16 * nvb}-column tiles")
    assert nvb > 1
    x = inputs.random_prefill(82, lengths, H=H, dk=d, dv=d, dtype=dtype, perkey=perkey,
                              chunk=chunk, prenorm=not l2, with_init=init)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    e_o, e_s = oracle.rel_err(o, o_ref), oracle.rel_err(pool, s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= BAR[dtype] and e_s <= BAR[dtype]


@pytest.mark.parametrize("dtype,perkey", [(torch.bfloat16, False), (torch.float32, True)])
def test_wide_tiles_checkpoints(dtype, perkey):
    """Checkpoints at chunk boundaries in some of 64 sequences x 4 heads: exported states vs
    the oracle's prefix states; outputs and final states bit-identical to the call without
    checkpoints."""
    d, chunk, H = 128, 64, 4
    lengths = _lengths(83, 64, 300)
    lengths[1], lengths[2] = 300, 64
    n = len(lengths)
    assert tile_width(dtype, n * H, d) > 1
    say(f"case wide-tile checkpoints {dtype} perkey={perkey}")
    x = inputs.random_prefill(84, lengths, H=H, dk=d, dv=d, dtype=dtype, perkey=perkey,
                              chunk=chunk, with_init=True)
    free = iter(range(n, n + 64))
    spec = [[] for _ in range(n)]
    spec[1] = [(chunk, next(free)), (3 * chunk, next(free)), (300, next(free))]
    spec[2] = [(64, next(free))]
    spec[5] = [(chunk, next(free))]
    n_slots = n + sum(len(e) for e in spec)
    pool0 = torch.randn(n_slots, H, d, d, generator=torch.Generator().manual_seed(6))
    pool0[:n] = x.init_states
    slots = torch.arange(n, dtype=torch.int32)
    has_init = torch.ones(n, dtype=torch.int32)
    o, pool = run_ckpt(x, pool0.clone(), slots, has_init, spec, chunk)
    o_plain, pool_plain = run_prefill(x)
    assert torch.equal(o, o_plain) and torch.equal(pool[:n], pool_plain)
    bar = BAR[dtype]
    o_ref, s_ref = oracle_prefill(x)
    assert oracle.rel_err(o, o_ref) <= bar and oracle.rel_err(pool[:n], s_ref) <= bar
    for i, entries in enumerate(spec):
        if not entries:
            continue
        stored = expected_stored(entries, lengths[i], chunk)
        want = [p for (p, _), st in zip(entries, stored) if st]
        ref = oracle_prefix_states(x, i, want, x.init_states[i])
        for (p, s), st in zip(entries, stored):
            if st:
                e = oracle.rel_err(pool[s], ref[p])
                say(f"   seq {i} p={p}: rel err {e:.2e}")
                assert e <= bar
            else:
                assert torch.equal(pool[s], pool0[s])


@pytest.mark.parametrize("dtype,perkey", [(torch.bfloat16, False), (torch.bfloat16, True),
                                          (torch.float32, False)])
def test_wide_tiles_conv_fused(dtype, perkey):
    """Conv-fused prefill of 64 sequences x 4 heads (v after the convolution goes through the
    workspace to the scan, which forms U), with conv histories and initial states for half of
    them: outputs and final states vs the oracle."""
    d, H, W = 64, 4, 4
    lengths = _lengths(85, 64, 120)
    n = len(lengths)
    assert tile_width(dtype, n * H, d) > 1
    say(f"case wide-tile conv prefill {dtype} perkey={perkey}")
    x = inputs.conv_prefill(86, lengths, H, d, width=W, dtype=dtype, perkey=perkey)
    CH = 3 * H * d
    has = [i % 2 for i in range(n)]
    cs0 = torch.zeros(n, CH, W - 1, dtype=dtype)
    pool0 = torch.zeros(n, H, d, d)
    hist_rows, init = [], torch.zeros(n, H, d, d)
    for i in range(n):
        if has[i]:
            cs0[i] = x.conv_hist[i]
            pool0[i] = x.init_states[i]
            init[i] = x.init_states[i]
            hist_rows.append(x.conv_hist[i].T)
        else:
            hist_rows.append(torch.zeros(W - 1, CH, dtype=dtype))
    slots = torch.arange(n, dtype=torch.int32)
    o, pool, _ = run_fused(x, pool0, slots, torch.tensor(has, dtype=torch.int32), cs0,
                           chunk=64)
    o_ref, s_ref = oracle_conv_prefill(x, hist_rows, init)
    e_o, e_s = oracle.rel_err(o, o_ref), oracle.rel_err(pool, s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= BAR[dtype] and e_s <= BAR[dtype]


def test_narrow_and_wide_tiles_agree():
    """The same sequence alone (16-column tiles: U and Q_in from the prep) and inside a batch
    of 64 (128-column tiles: U formed by the scan, q read by the scan): both within the bar
    of the oracle and of each other."""
    d, H = 128, 4
    lengths = _lengths(87, 64, 200)
    lengths[7] = 333
    x = inputs.random_prefill(88, lengths, H=H, dk=d, dv=d, with_init=True)
    assert tile_width(torch.bfloat16, 64 * H, d) == 8 and tile_width(torch.bfloat16, H, d) == 1
    say("case narrow vs wide tiles, sequence 7 of 64")
    o, pool = run_prefill(x)
    a, b = int(x.cu_seqlens[7]), int(x.cu_seqlens[8])
    x1 = inputs.PrefillInputs(q=x.q[a:b], k=x.k[a:b], v=x.v[a:b], g=x.g[a:b],
                              beta=x.beta[a:b], cu_seqlens=torch.tensor([0, b - a],
                                                                        dtype=torch.int32),
                              init_states=x.init_states[7:8], chunk=x.chunk, scale=x.scale,
                              qk_l2norm=x.qk_l2norm)
    o1, pool1 = run_prefill(x1)
    o_ref, s_ref = oracle_prefill(x1)
    for oo, pp in ((o[a:b], pool[7:8]), (o1, pool1)):
        assert oracle.rel_err(oo, o_ref) <= 1e-2 and oracle.rel_err(pp, s_ref) <= 1e-2
    e = oracle.rel_err(o[a:b], o1)
    say(f"   narrow vs wide: rel diff o={e:.2e}")
    assert e <= 1e-2
