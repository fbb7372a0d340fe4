"""Conv-fused chunked prefill on the GPU, through the C ABI.

Three kinds of check:
  - bit-identity with the two-launch path it replaces (gdn_conv1d_silu into three planes,
    then gdn_prefill_chunked): same fp32 tap order and SiLU, same rounding to the element
    type, then the same prep and scan;
  - parity with the fp64 oracle (oracle.conv1d_silu, then oracle.recurrence), including conv
    histories read from a conv-state pool; a history is checked as the first width-1 rows of
    a longer sequence (the convolution is causal, so the outputs after them are the same);
  - the conv-state pool after the call, a copy checked bit for bit, and a prefill followed by
    fused decode steps against the oracle over the whole sequence.
Bars: max|x - ref| / max|ref| <= 1e-4 (fp32 inputs) or 1e-2 (bf16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.gates import kda_forget_log, sigmoid
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, say, to_dev

pytestmark = pytest.mark.gpu


def planes(y, H, d):
    """[T, 3 H d] (or a [3, T, H d] plane stack) -> q, k, v as [T, H, d]."""
    if y.dim() == 3:
        return [y[p].reshape(-1, H, d).contiguous() for p in range(3)]
    HD = H * d
    return [y[:, p * HD:(p + 1) * HD].reshape(-1, H, d).contiguous() for p in range(3)]


def run_fused(x, pool0, slots, has_init=None, conv_state=None, chunk=64):
    """Returns (o, pool, conv_state) on the CPU."""
    X, w, g, b, cu, pd, sd, hi = to_dev(x.x, x.conv_w, x.g, x.beta, x.cu_seqlens, pool0.clone(),
                                        slots, has_init)
    cs = None if conv_state is None else conv_state.clone().to(DEV)
    o = gdn.gdn_prefill_chunked_conv(X, w, g, b, cu, chunk, pd, sd, conv_state=cs,
                                     has_init=hi, scale=x.scale, qk_l2norm=x.qk_l2norm)
    torch.cuda.synchronize()
    return o.cpu(), pd.cpu(), None if cs is None else cs.cpu()


def run_unfused(x, pool0, slots, chunk=64):
    X, w, g, b, cu, pd, sd = to_dev(x.x, x.conv_w, x.g, x.beta, x.cu_seqlens, pool0.clone(),
                                    slots)
    y = gdn.gdn_conv1d_silu(X, w, cu, planes=3)
    q, k, v = planes(y, x.H, x.d)
    o = gdn.gdn_prefill_chunked(q, k, v, g, b, cu, chunk, pd, sd, scale=x.scale,
                                qk_l2norm=x.qk_l2norm)
    torch.cuda.synchronize()
    return o.cpu(), pd.cpu()


def extended(x, hist_rows):
    """Each sequence's raw rows preceded by width-1 history rows (hist_rows[n] [W-1, CH], or
    zeros), packed; returns (rows, cu of the extended sequences)."""
    W1 = x.conv_w.shape[1] - 1
    cu = x.cu_seqlens.tolist()
    rows, ecu = [], [0]
    for n in range(len(cu) - 1):
        rows.append(hist_rows[n].to(torch.float64))
        rows.append(x.x[cu[n]:cu[n + 1]].to(torch.float64))
        ecu.append(ecu[-1] + W1 + cu[n + 1] - cu[n])
    return torch.cat(rows, 0), torch.tensor(ecu, dtype=torch.int32)


def oracle_conv_prefill(x, hist_rows, init):
    """fp64: convolution over the history-extended sequences, history outputs dropped, then
    the recurrence from `init` ([n, H, d, d], zeros = no initial state)."""
    W1 = x.conv_w.shape[1] - 1
    rows, ecu = extended(x, hist_rows)
    y = oracle.conv1d_silu(rows, x.conv_w, ecu)
    keep = np.concatenate([np.arange(int(ecu[n]) + W1, int(ecu[n + 1]))
                           for n in range(len(ecu) - 1)]).astype(np.int64)
    q, k, v = planes(torch.from_numpy(y[keep]), x.H, x.d)
    return oracle.recurrence(q, k, v, x.g, x.beta, x.cu_seqlens, scale=x.scale,
                             l2norm=x.qk_l2norm, init_states=init)


BITWISE = [
    # (dtype, d, chunk, perkey, width)
    (torch.bfloat16, 128, 64, True, 4),
    (torch.bfloat16, 128, 64, False, 4),
    (torch.bfloat16, 64, 32, True, 3),
    (torch.bfloat16, 16, 16, False, 2),
    (torch.float32, 32, 16, True, 4),
    (torch.float32, 128, 64, False, 3),
    (torch.float32, 16, 64, True, 2),
]


@pytest.mark.parametrize("dtype,d,chunk,perkey,W", BITWISE)
def test_fused_equals_unfused_bitwise(dtype, d, chunk, perkey, W):
    """Ragged lengths around the conv width and the chunk (0 .. 3 tokens, a chunk and a
    tail), no history: o and final states bit-identical to conv1d_silu + prefill."""
    lengths = [0, 1, 2, 3, 150, chunk, 77, 17]
    say(f"case conv-prefill bitwise {dtype} d={d} C={chunk} perkey={perkey} W={W}")
    H = 3
    x = inputs.conv_prefill(40, lengths, H, d, width=W, dtype=dtype, perkey=perkey)
    n = len(lengths)
    pool0 = torch.zeros(n, H, d, d)
    slots = torch.arange(n, dtype=torch.int32)
    o, pool, _ = run_fused(x, pool0, slots, chunk=chunk)
    o_u, pool_u = run_unfused(x, pool0, slots, chunk=chunk)
    assert torch.equal(o, o_u)
    assert torch.equal(pool, pool_u)


def test_fused_equals_unfused_many_sequences():
    """70 sequences of 0..40 tokens (the per-sequence chunk table comes from its own pass
    above 64 sequences)."""
    say("case conv-prefill bitwise, 70 short sequences")
    g = torch.Generator().manual_seed(41)
    lengths = torch.randint(0, 41, (70,), generator=g).tolist()
    H, d = 2, 64
    x = inputs.conv_prefill(42, lengths, H, d, width=4)
    n = len(lengths)
    pool0 = torch.zeros(n, H, d, d)
    slots = torch.arange(n, dtype=torch.int32)
    o, pool, _ = run_fused(x, pool0, slots, chunk=16)
    o_u, pool_u = run_unfused(x, pool0, slots, chunk=16)
    assert torch.equal(o, o_u) and torch.equal(pool, pool_u)


def test_fused_equals_unfused_full_size_kda():
    """The KDA varlen workload at full size (8 sequences, T ~ 49k, H=32, d=128, chunk 64,
    width 4, bf16): the fused prefill is bit-identical to conv1d_silu + prefill."""
    say("case conv-prefill bitwise, full-size KDA varlen batch")
    kv = inputs.kda_varlen_config(0)
    x = inputs.ConvPrefillInputs(x=kv.x, conv_w=kv.conv_w, g=kv.g, beta=kv.beta,
                                 cu_seqlens=kv.cu_seqlens, conv_hist=None, init_states=None,
                                 H=kv.H, d=kv.d, scale=kv.scale, qk_l2norm=True)
    n = kv.cu_seqlens.numel() - 1
    pool0 = torch.zeros(n, kv.H, kv.d, kv.d)
    slots = torch.arange(n, dtype=torch.int32)
    o, pool, _ = run_fused(x, pool0, slots, chunk=kv.chunk)
    o_u, pool_u = run_unfused(x, pool0, slots, chunk=kv.chunk)
    say(f"   T={x.x.shape[0]}")
    assert torch.equal(o, o_u) and torch.equal(pool, pool_u)


@pytest.mark.parametrize("dtype,d,chunk,perkey,W", [
    (torch.bfloat16, 128, 64, True, 4), (torch.bfloat16, 64, 16, False, 3),
    (torch.float32, 32, 32, True, 2), (torch.float32, 64, 64, False, 4),
])
def test_history_and_state_vs_oracle(dtype, d, chunk, perkey, W):
    """Sequences with and without conv history and initial state, one without a slot:
    outputs and final states vs the oracle; the conv-state pool afterwards holds each
    sequence's last width-1 raw rows (history rows where the sequence is shorter), bit for
    bit, and is untouched elsewhere."""
    lengths = [150, 1, 2, 0, 77, chunk, 33]
    has = [1, 1, 0, 1, 1, 0, 0]
    slot_of = [0, 2, 3, 5, 6, 7, -1]
    say(f"case conv-prefill history {dtype} d={d} C={chunk} perkey={perkey} W={W}")
    H, n_slots = 2, 9
    x = inputs.conv_prefill(43, lengths, H, d, width=W, dtype=dtype, perkey=perkey)
    n = len(lengths)
    CH = 3 * H * d
    gen = torch.Generator().manual_seed(44)
    cs0 = torch.randn(n_slots, CH, W - 1, generator=gen).to(dtype)
    pool0 = torch.randn(n_slots, H, d, d, generator=gen) / d ** 0.5
    hist_rows, init = [], torch.zeros(n, H, d, d)
    for i, s in enumerate(slot_of):
        if s >= 0:
            cs0[s] = x.conv_hist[i]
            pool0[s] = x.init_states[i]
        if s >= 0 and has[i]:
            hist_rows.append(x.conv_hist[i].T)
            init[i] = x.init_states[i]
        else:
            hist_rows.append(torch.zeros(W - 1, CH, dtype=dtype))
    slots = torch.tensor(slot_of, dtype=torch.int32)
    has_init = torch.tensor(has, dtype=torch.int32)
    o, pool, cs = run_fused(x, pool0, slots, has_init, cs0, chunk=chunk)
    o_ref, s_ref = oracle_conv_prefill(x, hist_rows, init)
    bar = BAR[dtype]
    assert oracle.rel_err(o, o_ref) <= bar
    for i, s in enumerate(slot_of):
        if s >= 0:
            assert oracle.rel_err(pool[s], s_ref[i]) <= bar, i
    rows, ecu = extended(x, hist_rows)
    touched = set()
    for i, s in enumerate(slot_of):
        if s < 0:
            continue
        touched.add(s)
        last = rows[int(ecu[i + 1]) - (W - 1):int(ecu[i + 1])]  # [W-1, CH], oldest first
        assert torch.equal(cs[s].to(torch.float64), last.T.contiguous()), i
    for s in range(n_slots):
        if s not in touched:
            assert torch.equal(cs[s], cs0[s]) and torch.equal(pool[s], pool0[s]), s


def test_prefill_then_fused_decode_vs_oracle():
    """A KDA layer end to end: conv-fused prefill of 3 prompts from fresh slots, then 3
    fused decode steps that read the conv states and states the prefill left. The gates are
    the KDA formula in both phases. Decode outputs and final states vs the oracle over the
    whole token sequence."""
    say("case conv-prefill -> fused decode handoff")
    H, d, W, n_dec = 2, 64, 4, 3
    lengths = [100, 5, 64]
    n, CH = len(lengths), 3 * H * d
    gen = torch.Generator().manual_seed(45)
    x = inputs.conv_prefill(46, lengths, H, d, width=W, dtype=torch.bfloat16, perkey=True)
    T = x.x.shape[0]
    A_log = torch.log(1.0 + 15.0 * torch.rand(H, generator=gen))
    dt = torch.randn(H, d, generator=gen) / 2
    fb = torch.randn(T + n * n_dec, H, d, generator=gen)   # prefill tokens, then decode rows
    wl = torch.randn(T + n * n_dec, H, generator=gen)
    xd = torch.randn(n_dec, n, CH, generator=gen).to(torch.bfloat16)
    lb = -5.0
    g_all = torch.from_numpy(kda_forget_log(fb.numpy(), dt.numpy(), A_log.numpy(), lb))
    b_all = torch.from_numpy(sigmoid(wl.numpy()))
    x.g = g_all[:T].float().contiguous()
    x.beta = b_all[:T].float().contiguous()
    slots = torch.arange(n, dtype=torch.int32)
    X, w, g, b, cu, sd = to_dev(x.x, x.conv_w, x.g, x.beta, x.cu_seqlens, slots)
    pool = torch.zeros(n, H, d, d, device=DEV)
    cs = torch.zeros(n, CH, W - 1, dtype=torch.bfloat16, device=DEV)
    gdn.gdn_prefill_chunked_conv(X, w, g, b, cu, 64, pool, sd, conv_state=cs, scale=x.scale,
                                 qk_l2norm=True)
    outs = []
    for s in range(n_dec):
        r = slice(T + s * n, T + (s + 1) * n)
        o = gdn.gdn_decode_fused(xd[s].to(DEV), w, cs, fb[r].contiguous().to(DEV),
                                 wl[r].contiguous().to(DEV), A_log.to(DEV), dt.to(DEV), lb,
                                 pool, sd, scale=x.scale, qk_l2norm=True)
        outs.append(o.cpu())
    torch.cuda.synchronize()
    # oracle: each sequence's prompt rows, then its decode rows, as one sequence
    cu_l = x.cu_seqlens.tolist()
    rows, gs, bs, cu2 = [], [], [], [0]
    for i in range(n):
        rows += [x.x[cu_l[i]:cu_l[i + 1]], xd[:, i]]
        dec = [T + s * n + i for s in range(n_dec)]
        gs += [g_all[cu_l[i]:cu_l[i + 1]], g_all[dec]]
        bs += [b_all[cu_l[i]:cu_l[i + 1]], b_all[dec]]
        cu2.append(cu2[-1] + lengths[i] + n_dec)
    cu2 = torch.tensor(cu2, dtype=torch.int32)
    y = oracle.conv1d_silu(torch.cat(rows, 0), x.conv_w, cu2)
    q, k, v = planes(torch.from_numpy(y), H, d)
    o_ref, s_ref = oracle.recurrence(q, k, v, torch.cat(gs, 0), torch.cat(bs, 0), cu2,
                                     scale=x.scale, l2norm=True)
    for s in range(n_dec):
        idx = [int(cu2[i]) + lengths[i] + s for i in range(n)]
        e = oracle.rel_err(outs[s], o_ref[idx])
        say(f"   decode step {s}: rel err {e:.2e}")
        assert e <= 1e-2
    assert oracle.rel_err(pool.cpu(), s_ref) <= 1e-2


def test_zero_tokens_keep_or_clear_the_histories():
    """Three empty sequences (total_tokens = 0): the raw projection is never read (x may be
    empty); a sequence with has_init keeps its state and conv window, one without gets the
    zero state and a zero window, a slotless one touches nothing."""
    say("case conv-prefill, zero tokens")
    H, d, W, n_slots = 2, 32, 3, 5
    CH = 3 * H * d
    gen = torch.Generator().manual_seed(47)
    pool0 = torch.randn(n_slots, H, d, d, generator=gen)
    cs0 = torch.randn(n_slots, CH, W - 1, generator=gen).to(torch.bfloat16)
    x = torch.empty(0, CH, dtype=torch.bfloat16, device=DEV)
    w = (torch.randn(CH, W, generator=gen) / 2).to(DEV)
    g = torch.empty(0, H, d, device=DEV)
    b = torch.empty(0, H, device=DEV)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    slots = torch.tensor([1, 3, -1], dtype=torch.int32, device=DEV)
    has = torch.tensor([1, 0, 1], dtype=torch.int32, device=DEV)
    pool, cs = pool0.clone().to(DEV), cs0.clone().to(DEV)
    o = gdn.gdn_prefill_chunked_conv(x, w, g, b, cu, 64, pool, slots, conv_state=cs,
                                     has_init=has, scale=0.1, qk_l2norm=True)
    torch.cuda.synchronize()
    pool, cs = pool.cpu(), cs.cpu()
    assert o.numel() == 0
    assert torch.equal(pool[1], pool0[1]) and torch.equal(cs[1], cs0[1])
    assert torch.equal(pool[3], torch.zeros_like(pool[3])) and torch.equal(cs[3], torch.zeros_like(cs[3]))
    for s in (0, 2, 4):
        assert torch.equal(pool[s], pool0[s]) and torch.equal(cs[s], cs0[s]), s
