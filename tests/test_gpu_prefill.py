"""Chunked prefill on the GPU vs the fp64 oracle, element by element, through the C ABI.

Bars (per tensor, max|x - ref| / max|ref|): 1e-4 for fp32 inputs, 1e-2 for bf16 inputs, on
outputs and final states.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, oracle_prefill, run_prefill, say, to_dev

pytestmark = pytest.mark.gpu


def _check(x, o, pool, o_ref, s_ref, bar=None, slots=None):
    bar = bar or BAR[x.dtype]
    e_o = oracle.rel_err(o, o_ref)
    sl = slots if slots is not None else torch.arange(x.n_seqs)
    e_s = oracle.rel_err(pool[sl.long()], s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e} (bar {bar:g})")
    assert np.isfinite(o.float().numpy()).all()
    assert e_o <= bar and e_s <= bar


def test_tiny_gdn_fp32():
    """Tiny GDN: T=64, H=1, d=16, chunk 16, fp32, zero initial state."""
    say("case tiny fp32 T=64 d=16 C=16")
    x = inputs.tiny_config(0)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


CASES = [
    # (dtype, d, chunk, perkey, lengths, init, l2norm)
    (torch.float32, 16, 16, False, [64], False, False),
    (torch.float32, 32, 32, True, [1, 31, 70], True, False),
    (torch.float32, 64, 64, False, [129, 5], True, True),
    (torch.float32, 128, 64, True, [100], True, False),
    (torch.bfloat16, 16, 16, True, [17, 64, 3], True, True),
    (torch.bfloat16, 16, 32, False, [50, 33], True, False),
    (torch.bfloat16, 32, 32, False, [65, 96], False, False),
    (torch.bfloat16, 64, 16, True, [200], True, False),
    (torch.bfloat16, 64, 64, False, [1, 2, 63, 64, 65], True, True),
    (torch.bfloat16, 128, 64, False, [300, 1, 77], True, False),
    (torch.bfloat16, 128, 64, True, [191, 64], True, True),
    (torch.bfloat16, 128, 32, True, [150], False, False),
    (torch.bfloat16, 128, 16, False, [90, 40], True, False),
]


@pytest.mark.parametrize("dtype,d,chunk,perkey,lengths,init,l2", CASES)
def test_prefill_vs_oracle(dtype, d, chunk, perkey, lengths, init, l2):
    say(f"case prefill {dtype} d={d} C={chunk} perkey={perkey} lens={lengths} init={init} l2={l2}")
    x = inputs.random_prefill(11, lengths, H=3, dk=d, dv=d, dtype=dtype, perkey=perkey,
                              chunk=chunk, prenorm=not l2, with_init=init)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


@pytest.mark.parametrize("nseq,dtype,perkey", [(48, torch.bfloat16, True),
                                               (48, torch.float32, False),
                                               (64, torch.bfloat16, False),
                                               (64, torch.float32, True)])
def test_many_sequences_wide_value_tiles(nseq, dtype, perkey):
    """Enough (sequence, head) units that the scan gives each workgroup several 16-column
    value tiles: 48 (two tiles) or 64 (four tiles) ragged sequences x 4 heads at d = 64."""
    say(f"case many sequences n={nseq} {dtype} perkey={perkey}")
    lengths = torch.randint(0, 140, (nseq,), generator=torch.Generator().manual_seed(21)).tolist()
    x = inputs.random_prefill(21, lengths, H=4, dk=64, dv=64, dtype=dtype, perkey=perkey,
                              with_init=True)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


@pytest.mark.parametrize("nseq", [65, 150])
def test_more_sequences_than_one_wave(nseq):
    """Past 64 sequences the per-sequence first-chunk table comes from its own pass instead
    of being formed inside each wave: ragged lengths (empty ones included), H = 2, d = 32."""
    say(f"case prefill {nseq} sequences")
    lengths = torch.randint(0, 100, (nseq,), generator=torch.Generator().manual_seed(22)).tolist()
    lengths[3] = 0
    x = inputs.random_prefill(23, lengths, H=2, dk=32, dv=32, chunk=32, with_init=True)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


@pytest.mark.parametrize("perkey", [False, True])
def test_chunk_size_invariance(perkey):
    """The chunk size is an execution choice: C = 16, 32, 64 give the same result."""
    say(f"case chunk invariance perkey={perkey}")
    x = inputs.random_prefill(12, [333, 45], H=2, dk=128, dv=128, perkey=perkey, with_init=True)
    outs = [run_prefill(x, chunk=c) for c in (16, 32, 64)]
    o_ref, s_ref = oracle_prefill(x)
    for o, pool in outs:
        _check(x, o, pool, o_ref, s_ref)


def test_split_prefill_handoff_and_decode_continuation():
    """Handbook split-prefill: 20 | 25 | 19 tokens with the state handed over through the pool,
    then decode steps, equals one-shot prefill of all 64 + 8 tokens."""
    say("case split handoff")
    T = 72
    x = inputs.random_prefill(13, [T], H=4, dk=128, dv=128)
    o_ref, s_ref = oracle_prefill(x)
    pool = torch.zeros((2, 4, 128, 128), device=DEV)
    slots = torch.tensor([1], dtype=torch.int32, device=DEV)
    outs = []
    for i, (a, b) in enumerate(((0, 20), (20, 45), (45, 64))):
        q, k, v, g, be = to_dev(x.q[a:b], x.k[a:b], x.v[a:b], x.g[a:b], x.beta[a:b])
        cu = torch.tensor([0, b - a], dtype=torch.int32, device=DEV)
        hi = torch.tensor([1 if i else 0], dtype=torch.int32, device=DEV)
        outs.append(gdn.gdn_prefill_chunked(q, k, v, g, be, cu, 64, pool, slots, has_init=hi,
                                            scale=x.scale).cpu())
    for t in range(64, T):
        q, k, v, g, be = to_dev(*(z[t:t + 1] for z in (x.q, x.k, x.v, x.g, x.beta)))
        outs.append(gdn.gdn_decode_step(q, k, v, g, be, pool, slots, scale=x.scale).cpu())
    torch.cuda.synchronize()
    o = torch.cat(outs)
    assert oracle.rel_err(o, o_ref) <= 1e-2
    assert oracle.rel_err(pool.cpu()[1], s_ref[0]) <= 1e-2
    assert torch.all(pool.cpu()[0] == 0)


def test_per_key_equal_channels_matches_scalar_gate():
    say("case per-key equal channels")
    x = inputs.random_prefill(14, [200, 37], H=2, dk=64, dv=64, with_init=True)
    o1, p1 = run_prefill(x)
    x.g = x.g[:, :, None].expand(-1, -1, 64).contiguous()
    o2, p2 = run_prefill(x)
    assert oracle.rel_err(o2, o1) <= 1e-2 and oracle.rel_err(p2, p1) <= 1e-2


def test_per_key_strong_decay_no_overflow():
    """Appendix 1 stress: per-key log gate -5 on every channel and step (the pages' lower
    bound): the in-chunk cumulative gate reaches -320; results stay finite and match."""
    say("case per-key g=-5 stress")
    x = inputs.random_prefill(15, [256], H=2, dk=128, dv=128, perkey=True, with_init=True)
    x.g = torch.full_like(x.g, -5.0)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


def test_slots_untouched_noslot_and_empty_sequences():
    """Pool slots not named stay bit-identical; a sequence with slot -1 starts from zero and
    stores nothing; empty sequences store their initial (or zero) state."""
    say("case slots / no-slot / empty")
    x = inputs.random_prefill(16, [40, 0, 70, 0], H=2, dk=64, dv=64, with_init=True)
    pool = torch.randn(6, 2, 64, 64)
    slots = torch.tensor([4, 1, -1, 2], dtype=torch.int32)
    has_init = torch.tensor([1, 1, 1, 0], dtype=torch.int32)
    init = torch.stack([pool[4], pool[1], torch.zeros(2, 64, 64), torch.zeros(2, 64, 64)])
    o, after = run_prefill(x, pool=pool.clone(), slots=slots, has_init=has_init)
    o_ref, s_ref = oracle_prefill(x, init=init)
    assert oracle.rel_err(o, o_ref) <= 1e-2
    assert oracle.rel_err(after[4], s_ref[0]) <= 1e-2
    assert torch.equal(after[1], pool[1])               # empty sequence, has_init
    assert torch.all(after[2] == 0)                     # empty sequence, zero init
    for untouched in (0, 3, 5):
        assert torch.equal(after[untouched], pool[untouched])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_degenerate_no_write_no_decay(dtype):
    """beta = 0 and g = 0: nothing is written and nothing decays, so the state stays exactly
    the initial state and every output is scale * S_0^T q (the beta = 0 closed form)."""
    say(f"case degenerate beta=0 g=0 {dtype}")
    x = inputs.random_prefill(24, [200, 64, 1], H=2, dk=64, dv=64, dtype=dtype, with_init=True)
    x.beta = torch.zeros_like(x.beta)
    x.g = torch.zeros_like(x.g)
    o, pool = run_prefill(x)
    assert torch.equal(pool, x.init_states.float())
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


def test_zero_queries_give_zero_outputs():
    say("case zero queries")
    x = inputs.random_prefill(25, [150, 33], H=2, dk=128, dv=128, with_init=True)
    x.q = torch.zeros_like(x.q)
    o, pool = run_prefill(x)
    assert torch.all(o == 0)
    o_ref, s_ref = oracle_prefill(x)
    assert oracle.rel_err(pool, s_ref) <= 1e-2


def test_long_sequence_many_chunks():
    """One 65536-token sequence (1024 chunks of 64), H = 2, d = 64, bf16, with an initial
    state: outputs and final state against the oracle."""
    say("case long sequence T=65536")
    x = inputs.random_prefill(26, [65536], H=2, dk=64, dv=64, with_init=True)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


def test_deterministic():
    say("case determinism")
    x = inputs.random_prefill(17, [500, 300], H=4, dk=128, dv=128, perkey=True)
    o1, p1 = run_prefill(x)
    o2, p2 = run_prefill(x)
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


def test_prefill_config_full_size():
    """GDN chunked prefill at its full size: B=1, H=16, T=8192, d=128, chunk 64, bf16."""
    say("case prefill full size T=8192 H=16")
    x = inputs.prefill_config(0)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


def test_prefill_batch_32x2048_full():
    """A serving-style batch at full size: 32 sequences x 2048 tokens, H=16, d=128, chunk 64,
    bf16 (the per-(sequence, head) scan runs 8 value tiles per workgroup here). Every output
    and final state against the oracle."""
    say("case prefill batch 32 x 2048, H=16")
    x = inputs.prefill_batch_config(0)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)


def test_kda_varlen_conv_fused_all_heads():
    """KDA-style varlen prefill at full size, as the benchmark times it: 8 sequences of 1k-8k
    tokens, H=32, d=128, bf16, the causal conv1d + SiLU fused into the prefill, in-kernel L2
    norm, per-key gate. Every output of every head and every final state against the oracle
    (fp64 convolution, then the fp64 recurrence); the standalone convolution's q, k, v planes
    against the oracle's convolution on every channel."""
    from test_gpu_conv_prefill import oracle_conv_prefill, planes, run_fused
    say("case KDA varlen full size, conv fused, all heads")
    kv = inputs.kda_varlen_config(0)
    H, d = kv.H, kv.d
    n = kv.cu_seqlens.numel() - 1
    x = inputs.ConvPrefillInputs(x=kv.x, conv_w=kv.conv_w, g=kv.g, beta=kv.beta,
                                 cu_seqlens=kv.cu_seqlens, conv_hist=None, init_states=None,
                                 H=H, d=d, scale=kv.scale, qk_l2norm=True)
    o, pool, _ = run_fused(x, torch.zeros(n, H, d, d), torch.arange(n, dtype=torch.int32),
                           chunk=kv.chunk)
    xd, wd, cud = to_dev(kv.x, kv.conv_w, kv.cu_seqlens)
    qkv = gdn.gdn_conv1d_silu(xd, wd, cud, planes=3).cpu()
    torch.cuda.synchronize()
    say(f"   GPU done (T={kv.x.shape[0]}); oracle over all {n * H} (sequence, head) units")
    y = torch.from_numpy(oracle.conv1d_silu(kv.x, kv.conv_w, kv.cu_seqlens))
    for got, ref in zip(planes(qkv, H, d), planes(y, H, d)):
        assert oracle.rel_err(got, ref) <= 1e-2
    del y, qkv
    hist = [torch.zeros(3, 3 * H * d, dtype=kv.x.dtype) for _ in range(n)]
    o_ref, s_ref = oracle_conv_prefill(x, hist, torch.zeros(n, H, d, d))
    e_o = oracle.rel_err(o, o_ref)
    e_s = oracle.rel_err(pool, s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert np.isfinite(o.float().numpy()).all()
    assert e_o <= 1e-2 and e_s <= 1e-2


@pytest.mark.parametrize("lengths,H", [([8192], 2), ("many", 4)])
def test_value_scale_equivariance(lengths, H):
    """With a zero initial state the outputs and final states are linear in v, and every
    operation on v-derived quantities (the fp32 arithmetic, RNE to bf16, U in fp32) commutes
    with scaling by a power of two. So v * 2^10 and v * 2^-10 must give outputs and states
    scaled exactly, bit for bit. 'many' is 64 ragged sequences, whose scan forms U itself
    from v; one long sequence reads the prep's U."""
    if lengths == "many":
        lengths = torch.randint(1, 200, (64,), generator=torch.Generator().manual_seed(71)).tolist()
    say(f"case value-scale equivariance, {len(lengths)} sequences, H={H}")
    x = inputs.random_prefill(72, lengths, H=H, dk=128, dv=128)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    _check(x, o, pool, o_ref, s_ref)
    v0 = x.v
    for sc in (2.0 ** 10, 2.0 ** -10):
        x.v = (v0.float() * sc).to(v0.dtype)
        o2, pool2 = run_prefill(x)
        assert torch.equal(o2.float(), o.float() * sc)
        assert torch.equal(pool2, pool * sc)
