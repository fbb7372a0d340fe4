"""Prefill under strong and abrupt decay, on the GPU vs the fp64 oracle, through the C ABI.

The per-key (KDA) gate's A and M need e^{G_i - G_j} per key channel. [LA-Infra] appendix
"附1. chunk内 A和M 的计算" splits it at a reference point for the off-diagonal 16x16 blocks and
computes the diagonal blocks directly; the gate contract is any finite g <= 0. These cases
reach cumulative decays far beyond fp32's exponent range inside one 16-token block:
  - g = -6 on every channel and step (90 nats across a block);
  - ordinary gates with single hard-forget tokens, g = -100, inside blocks;
  - g uniform in [-30, 0] (hundreds of nats across a block).
Each runs through the plain prefill, the checkpointing prefill and the conv-fused prefill,
against the oracle at the usual bars, and the plain prefill is also compared with the same
tokens fed one by one to the decode step. Scalar (GDN) gates take the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, oracle_prefill, run_prefill, say, to_dev
from test_gpu_checkpoint import expected_stored, oracle_prefix_states, run_ckpt
from test_gpu_conv_prefill import oracle_conv_prefill, run_fused

pytestmark = pytest.mark.gpu

KINDS = ["minus6", "hard_forget", "uniform30"]
HARD = [5, 37, 70, 127, 150, 201, 263]  # token positions given g = -100


def strong_gates(kind, g, seed):
    """Replace the log gates g ([T, H] or [T, H, d_k]) by one of the strong-decay kinds."""
    gen = torch.Generator().manual_seed(seed)
    if kind == "minus6":
        return torch.full_like(g, -6.0)
    if kind == "uniform30":
        return (-30.0 * torch.rand(g.shape, generator=gen)).to(g.dtype)
    out = g.clone()
    for t in HARD:
        if t < g.shape[0]:
            out[t] = -100.0
    return out


def _check(o, o_ref, pool, s_ref, bar, what):
    e_o = oracle.rel_err(o, o_ref)
    e_s = oracle.rel_err(pool, s_ref)
    say(f"   {what}: rel err o={e_o:.2e} S={e_s:.2e} (bar {bar:g})")
    assert np.isfinite(o.float().numpy()).all() and np.isfinite(pool.numpy()).all()
    assert e_o <= bar and e_s <= bar


PLAIN = [
    # (dtype, d, chunk, perkey)
    (torch.bfloat16, 128, 64, True),
    (torch.bfloat16, 128, 32, True),
    (torch.bfloat16, 64, 16, True),
    (torch.bfloat16, 128, 64, False),
    (torch.float32, 128, 64, True),
    (torch.float32, 32, 32, True),
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d,chunk,perkey", PLAIN)
def test_plain_prefill_strong_decay(kind, dtype, d, chunk, perkey):
    lengths = [300, 77, 16]
    say(f"case strong decay {kind} plain {dtype} d={d} C={chunk} perkey={perkey}")
    x = inputs.random_prefill(61, lengths, H=2, dk=d, dv=d, dtype=dtype, perkey=perkey,
                              chunk=chunk, with_init=True)
    x.g = strong_gates(kind, x.g, 62)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(o, o_ref, pool, s_ref, BAR[dtype], "prefill vs oracle")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("perkey", [True, False])
def test_prefill_equals_token_by_token_decode(kind, perkey):
    """The same 200 tokens through one prefill and through 200 decode steps (both on the
    GPU, both against the oracle, and against each other)."""
    say(f"case strong decay {kind} prefill == decode perkey={perkey}")
    T, H, d = 200, 2, 128
    x = inputs.random_prefill(63, [T], H=H, dk=d, dv=d, perkey=perkey, with_init=True)
    x.g = strong_gates(kind, x.g, 64)
    o_p, pool_p = run_prefill(x)
    pool = x.init_states.clone().float().to(DEV)
    slot = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = []
    for t in range(T):
        q, k, v, g, b = to_dev(*(z[t:t + 1] for z in (x.q, x.k, x.v, x.g, x.beta)))
        outs.append(gdn.gdn_decode_step(q, k, v, g, b, pool, slot, scale=x.scale))
    torch.cuda.synchronize()
    o_d = torch.cat(outs).cpu()
    pool_d = pool.cpu()
    o_ref, s_ref = oracle_prefill(x)
    _check(o_p, o_ref, pool_p, s_ref, 1e-2, "prefill vs oracle")
    _check(o_d, o_ref, pool_d, s_ref, 1e-2, "decode vs oracle")
    _check(o_p, o_d.float(), pool_p, pool_d, 2e-2, "prefill vs decode")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d,chunk", [(torch.bfloat16, 128, 64), (torch.float32, 64, 32)])
def test_checkpoint_prefill_strong_decay(kind, dtype, d, chunk):
    lengths = [300, 130]
    say(f"case strong decay {kind} ckpt {dtype} d={d} C={chunk}")
    H, n = 2, 2
    x = inputs.random_prefill(65, lengths, H=H, dk=d, dv=d, dtype=dtype, perkey=True,
                              chunk=chunk, with_init=True)
    x.g = strong_gates(kind, x.g, 66)
    spec = [[(chunk, 2), (2 * chunk, 3), (300, 4)], [(chunk, 5), (130, 6)]]
    n_slots = 7
    pool0 = torch.randn(n_slots, H, d, d, generator=torch.Generator().manual_seed(67))
    pool0[:n] = x.init_states
    slots = torch.arange(n, dtype=torch.int32)
    has_init = torch.ones(n, dtype=torch.int32)
    o, pool = run_ckpt(x, pool0.clone(), slots, has_init, spec, chunk)
    bar = BAR[dtype]
    o_ref, s_ref = oracle_prefill(x)
    _check(o, o_ref, pool[:n], s_ref, bar, "ckpt prefill vs oracle")
    for i, entries in enumerate(spec):
        stored = expected_stored(entries, lengths[i], chunk)
        want = [p for (p, _), st in zip(entries, stored) if st]
        ref = oracle_prefix_states(x, i, want, x.init_states[i])
        for (p, s), st in zip(entries, stored):
            assert st
            e = oracle.rel_err(pool[s], ref[p])
            say(f"   checkpoint seq {i} offset {p}: rel err {e:.2e}")
            assert np.isfinite(pool[s].numpy()).all() and e <= bar


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype,d,chunk,perkey", [(torch.bfloat16, 128, 64, True),
                                                  (torch.bfloat16, 64, 32, False),
                                                  (torch.float32, 32, 16, True)])
def test_conv_prefill_strong_decay(kind, dtype, d, chunk, perkey):
    lengths = [300, 3, 90]
    say(f"case strong decay {kind} conv-fused {dtype} d={d} C={chunk} perkey={perkey}")
    H = 2
    x = inputs.conv_prefill(68, lengths, H, d, width=4, dtype=dtype, perkey=perkey)
    x.g = strong_gates(kind, x.g, 69)
    n = len(lengths)
    pool0 = torch.zeros(n, H, d, d)
    slots = torch.arange(n, dtype=torch.int32)
    o, pool, _ = run_fused(x, pool0, slots, chunk=chunk)
    hist = [torch.zeros(3, 3 * H * d, dtype=dtype) for _ in range(n)]
    o_ref, s_ref = oracle_conv_prefill(x, hist, torch.zeros(n, H, d, d))
    _check(o, o_ref, pool, s_ref, BAR[dtype], "conv prefill vs oracle")
