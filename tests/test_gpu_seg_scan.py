"""Segmented scan on the GPU vs the fp64 oracle, through the C ABI.

With d_k = d_v = 64 or 128, C = 64 and few (sequence, head) units (value tiles at most half
the CU count), the scan cuts each sequence of n >= 40 chunks into k segments run at once
(k = 2 below 80 chunks, then min(K, n / 20); K = CUs / (units x d / 16), at most 8): the
first from the initial state, each later one from a zero state beside an identity run that yields the segment's
transition. A chain pass carries the state across the boundaries (S_{j+1} = P_j S_j +
Delta_j) and a combine pass adds (identity-run outputs) x (state at the segment's start) to
each later segment's outputs and forms the final state ([LA-Infra] "Linear Attention
Chunk-Wise": chunk states compose as S_C = Transition S_0 + Delta). These cases cover 2 to 8
segments, split and unsplit sequences in one call, ragged and empty sequences, initial
states, slots outside the pool, both gates, very strong decay, the in-kernel L2 norm and the
fused convolution, and fp32 inputs. Bars: max|x - ref| / max|ref| <= 1e-2 (bf16 inputs), 1e-4
(fp32 inputs).
"""
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, oracle_prefill, run_prefill, say
from test_gpu_conv_prefill import oracle_conv_prefill, run_fused

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def seg_active(H, n_seqs, T, perkey=False, d=128, dtype=BF):
    """True when the library sizes the workspace for the segmented scan for this call."""
    e = 2 if dtype == BF else 4
    plain = ((T + n_seqs * 63) // 64) * H * (
        64 * d * e * 2 + d * 64 * e + 64 * 64 * e
        + max(64 * d * 4, 64 * 64 * e + 64 * 4 + 64 * d * e + 64 * 4) + d * 4)
    need = gdn.gdn_prefill_workspace_bytes(H, d, d, dtype, perkey, n_seqs, T, 64)
    return need > plain + n_seqs * H * d * d * 14


def _check(x, o, pool, heads=None):
    o_ref, s_ref = oracle_prefill(x)
    e_o, e_s = oracle.rel_err(o, o_ref), oracle.rel_err(pool, s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= BAR[BF] and e_s <= BAR[BF]


@pytest.mark.parametrize("lengths,H,perkey,init,l2", [
    ([4096], 2, False, True, True),        # 64 chunks, K = 8: 2 segments
    ([3000], 4, True, True, False),        # ragged last chunk, per-key gate: 2 segments
    ([2560], 1, False, False, True),       # exactly 40 chunks: the shortest split
    ([9000, 0, 700, 2560], 2, False, True, True),  # K = 4: 4 segments, empty, 1, 2
    ([2222, 4500], 4, True, False, True),  # K = 4: unsplit (35 chunks), 2 segments
    ([5200, 5200, 1000], 3, False, True, True),  # 9 units, K = 3: 3, 3, unsplit
    ([8192], 1, False, True, True),        # 128 chunks: 6 segments
    ([12000], 1, True, True, True),        # 188 chunks: 8 segments (K), per-key gate
])
def test_segmented_vs_oracle(lengths, H, perkey, init, l2):
    T = sum(lengths)
    say(f"case segmented scan lengths={lengths} H={H} perkey={perkey} init={init} l2={l2}")
    assert seg_active(H, len(lengths), T, perkey)
    x = inputs.random_prefill(91, lengths, H=H, dk=128, dv=128, dtype=BF, perkey=perkey,
                              prenorm=not l2, with_init=init)
    o, pool = run_prefill(x)
    _check(x, o, pool)


@pytest.mark.parametrize("lengths,H,perkey", [
    ([8192], 2, False),          # K = 8: 6 segments
    ([3000, 6000], 4, True),     # K = 8: 2 and 4 segments, per-key gate
    ([5000, 5000], 16, False),   # 32 units, K = 2: the two-segment form and its prep order
])
def test_segmented_d64_vs_oracle(lengths, H, perkey):
    """d_k = d_v = 64: 4 value tiles per head, so the segments fit for twice the units."""
    T = sum(lengths)
    say(f"case segmented scan d=64 lengths={lengths} H={H} perkey={perkey}")
    assert seg_active(H, len(lengths), T, perkey, d=64)
    x = inputs.random_prefill(96, lengths, H=H, dk=64, dv=64, dtype=BF, perkey=perkey,
                              with_init=True)
    o, pool = run_prefill(x)
    _check(x, o, pool)


@pytest.mark.parametrize("lengths,H,d,perkey", [
    ([8192], 2, 128, False),      # K = 8: 6 segments
    ([3000, 6000], 4, 64, True),  # K = 8: 2 and 4 segments, per-key gate
    ([5000], 16, 128, True),      # K = 2
])
def test_segmented_fp32_vs_oracle(lengths, H, d, perkey):
    """fp32 inputs: the same segmented scan on fp32 MFMA throughout (the combine's L S_j
    product and the chain too), at the fp32 bar."""
    F32 = torch.float32
    T = sum(lengths)
    say(f"case segmented scan fp32 d={d} lengths={lengths} H={H} perkey={perkey}")
    assert seg_active(H, len(lengths), T, perkey, d=d, dtype=F32)
    x = inputs.random_prefill(97, lengths, H=H, dk=d, dv=d, dtype=F32, perkey=perkey,
                              with_init=True)
    o, pool = run_prefill(x)
    o_ref, s_ref = oracle_prefill(x)
    e_o, e_s = oracle.rel_err(o, o_ref), oracle.rel_err(pool, s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= BAR[F32] and e_s <= BAR[F32]


def test_segmented_slots_outside_pool_and_untouched_slots():
    """K = 5: a sequence of 4 segments, one of 2 whose slot is -1 (no state read or
    written) and an unsplit one whose slot is past the pool: outputs still match, the other
    pool slots stay bit-identical."""
    lengths = [5100, 2600, 1500]
    n, H = 3, 2
    assert seg_active(H, n, sum(lengths))
    say("case segmented scan with slots outside the pool")
    x = inputs.random_prefill(92, lengths, H=H, dk=128, dv=128, dtype=BF, with_init=True)
    pool0 = torch.randn(5, H, 128, 128, generator=torch.Generator().manual_seed(3))
    pool0[4] = x.init_states[0]
    slots = torch.tensor([4, -1, 7], dtype=torch.int32)  # 7 is past a 5-slot pool
    has_init = torch.tensor([1, 1, 1], dtype=torch.int32)
    o, pool = run_prefill(x, pool=pool0.clone(), slots=slots, has_init=has_init)
    init = torch.zeros(n, H, 128, 128)
    init[0] = x.init_states[0]
    o_ref, s_ref = oracle_prefill(x, init=init)
    e_o = oracle.rel_err(o, o_ref)
    e_s = oracle.rel_err(pool[4], s_ref[0])
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= BAR[BF] and e_s <= BAR[BF]
    assert torch.equal(pool[:4], pool0[:4])


@pytest.mark.parametrize("perkey", [False, True])
def test_segmented_strong_decay(perkey):
    """Gates at -6 on every step and a -100 token inside a block of the last of 4 segments:
    the transitions are then (near) zero and the chain and combine must still be exact."""
    lengths = [6000]
    H = 2
    say(f"case segmented scan with strong decay perkey={perkey}")
    x = inputs.random_prefill(93, lengths, H=H, dk=128, dv=128, dtype=BF, perkey=perkey,
                              with_init=True)
    g = torch.full_like(x.g, -6.0)
    g[5000] = -100.0
    x.g = g
    o, pool = run_prefill(x)
    _check(x, o, pool)


@pytest.mark.parametrize("d", [128, 64])
def test_segmented_conv_fused(d):
    """Conv-fused prefill of 2 sequences x 4 heads (4 and 2 segments), with a conv history
    and an initial state for one of them."""
    lengths = [6100, 2600]
    n, H, W = 2, 4, 4
    assert seg_active(H, n, sum(lengths), d=d)
    say(f"case segmented scan, conv-fused prefill d={d}")
    x = inputs.conv_prefill(94, lengths, H, d, width=W, dtype=BF, perkey=False)
    CH = 3 * H * d
    cs0 = torch.zeros(n, CH, W - 1, dtype=BF)
    cs0[0] = x.conv_hist[0]
    pool0 = torch.zeros(n, H, d, d)
    pool0[0] = x.init_states[0]
    init = torch.zeros(n, H, d, d)
    init[0] = x.init_states[0]
    hist_rows = [x.conv_hist[0].T, torch.zeros(W - 1, CH, dtype=BF)]
    o, pool, _ = run_fused(x, pool0, torch.arange(n, dtype=torch.int32),
                           torch.tensor([1, 0], dtype=torch.int32), cs0, chunk=64)
    o_ref, s_ref = oracle_conv_prefill(x, hist_rows, init)
    e_o, e_s = oracle.rel_err(o, o_ref), oracle.rel_err(pool, s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= BAR[BF] and e_s <= BAR[BF]


def test_segmented_against_one_segment():
    """The same call (2 segments) with a checkpoint list (which keeps the scan in one
    segment) and without: both within the bar of the oracle and of each other, and the
    segmented call is deterministic."""
    lengths = [3500]
    H = 2
    x = inputs.random_prefill(95, lengths, H=H, dk=128, dv=128, dtype=BF, with_init=True)
    say("case two-segment vs one-segment scan")
    o, pool = run_prefill(x)
    o2, pool2 = run_prefill(x)
    assert torch.equal(o, o2) and torch.equal(pool, pool2)
    q, k, v, g, b, cu = (t.to("cuda:0") for t in (x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens))
    pd = x.init_states.clone().float().to("cuda:0")
    ext = torch.randn(1, H, 128, 128).to("cuda:0")
    pool_ck = torch.cat([pd, ext])
    o1 = gdn.gdn_prefill_chunked_ckpt(
        q, k, v, g, b, cu, 64, pool_ck, torch.zeros(1, dtype=torch.int32, device="cuda:0"),
        torch.tensor([0, 1], dtype=torch.int32, device="cuda:0"),
        torch.tensor([3500], dtype=torch.int32, device="cuda:0"),
        torch.tensor([1], dtype=torch.int32, device="cuda:0"),
        has_init=torch.ones(1, dtype=torch.int32, device="cuda:0"), scale=x.scale,
        qk_l2norm=x.qk_l2norm).cpu()
    pool1 = pool_ck.cpu()
    torch.cuda.synchronize()
    _check(x, o, pool)
    _check(x, o1, pool1[:1])
    assert torch.equal(pool1[1], pool1[0])  # the checkpoint at the end is the final state
    e = oracle.rel_err(o, o1)
    say(f"   two vs one segment: rel diff o={e:.2e}")
    assert e <= 1e-2


def test_segmented_full_size_few_heads():
    """The call bench.py times as `prefill_few_heads` (same seeded inputs: one sequence of
    32768 tokens, H = 2, bf16, d = 128, chunk 64; 8 segments, 6 chain steps), every output
    and both heads' final states against the oracle."""
    say("case segmented scan at the few-heads bench size (32768 tokens, H=2)")
    x = inputs.random_prefill(7, [32768], H=2, dk=128, dv=128, dtype=BF)
    assert seg_active(2, 1, 32768)
    o, pool = run_prefill(x)
    _check(x, o, pool)


def test_segmented_full_size_few_heads_d64():
    """The call bench.py times as `prefill_few_heads_d64` (same seeded inputs: one sequence
    of 32768 tokens, H = 4, d_k = d_v = 64; 8 segments), every output and every head's final
    state against the oracle."""
    say("case segmented scan at the d=64 few-heads bench size (32768 tokens, H=4)")
    x = inputs.random_prefill(7, [32768], H=4, dk=64, dv=64, dtype=BF)
    assert seg_active(4, 1, 32768, d=64)
    o, pool = run_prefill(x)
    _check(x, o, pool)
