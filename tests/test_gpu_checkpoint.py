"""Prefill with internal checkpoints on the GPU vs the fp64 oracle, through the C ABI.

A checkpoint is the state after the first p tokens of a sequence. Its oracle value is the
sequential recurrence over those p tokens from the sequence's initial state, computed by
chaining oracle runs over the segments between consecutive checkpoints (the recurrence is
sequential, so handing the state from one segment to the next is exact). Bars as the other
prefill tests: max|x - ref| / max|ref| <= 1e-4 (fp32 inputs) or 1e-2 (bf16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, oracle_prefill, say, to_dev

pytestmark = pytest.mark.gpu


def expected_stored(entries, length, chunk):
    """Which checkpoint entries of one sequence are stored: offset usable (0 < p <= length,
    p a multiple of the chunk or the length) and not below an earlier entry's offset."""
    out, high = [], -1 << 30
    for p, _slot in entries:
        usable = 0 < p <= length and (p % chunk == 0 or p == length)
        out.append(usable and p >= high)
        high = max(high, p)
    return out


def oracle_prefix_states(x, n, positions, init):
    """fp64 states of sequence n after each of the sorted token counts in `positions`."""
    t0 = int(x.cu_seqlens[n])
    state = init[None].clone() if init is not None else None
    done, out = 0, {}
    for p in sorted(set(positions)):
        a, b = t0 + done, t0 + p
        cu = torch.tensor([0, p - done], dtype=torch.int32)
        _, s = oracle.recurrence(x.q[a:b], x.k[a:b], x.v[a:b], x.g[a:b], x.beta[a:b], cu,
                                 scale=x.scale, l2norm=x.qk_l2norm, init_states=state)
        out[p] = s[0]
        state = torch.from_numpy(s)
        done = p
    return out


def run_ckpt(x, pool, slots, has_init, spec, chunk):
    """spec: per sequence, a list of (offset, slot). Returns (o, pool) on the CPU."""
    cu_ck = [0]
    pos, sl = [], []
    for entries in spec:
        for p, s in entries:
            pos.append(p)
            sl.append(s)
        cu_ck.append(len(pos))
    q, k, v, g, b, cu, pd, sd, hi = to_dev(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool,
                                          slots, has_init)
    ck_cu, ck_pos, ck_sl = (torch.tensor(z, dtype=torch.int32, device=DEV)
                            for z in (cu_ck, pos, sl))
    o = gdn.gdn_prefill_chunked_ckpt(q, k, v, g, b, cu, chunk, pd, sd, ck_cu, ck_pos, ck_sl,
                                     has_init=hi, scale=x.scale, qk_l2norm=x.qk_l2norm)
    torch.cuda.synchronize()
    return o.cpu(), pd.cpu()


def run_plain(x, pool, slots, has_init, chunk):
    q, k, v, g, b, cu, pd, sd, hi = to_dev(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool,
                                          slots, has_init)
    o = gdn.gdn_prefill_chunked(q, k, v, g, b, cu, chunk, pd, sd, has_init=hi, scale=x.scale,
                                qk_l2norm=x.qk_l2norm)
    torch.cuda.synchronize()
    return o.cpu(), pd.cpu()


def ragged_spec(C, lengths, first_free):
    """Checkpoint lists that mix usable entries with every kind the kernel must skip."""
    s = iter(range(first_free, first_free + 64))
    L0, L1, L2, L3 = lengths[:4]
    return [
        # usable, between boundaries, null block, usable, the sequence end, past the end
        [(C, next(s)), (C + 5, next(s)), (2 * C, -1), (3 * C, next(s)), (L0, next(s)),
         (L0 + C, next(s))],
        [(L1, next(s))],                                 # a 1-token sequence: its end
        [(C, next(s)), (L2, next(s)), (L2, next(s))],    # equal offsets: both stored
        [(C, next(s)), (C // 2, next(s)), (2 * C, next(s))],  # below an earlier offset
        [(C, next(s))],                                  # empty sequence
    ]


CASES = [
    # (dtype, d, chunk, perkey)
    (torch.bfloat16, 128, 64, False),
    (torch.bfloat16, 128, 64, True),
    (torch.bfloat16, 64, 32, True),
    (torch.bfloat16, 16, 16, False),
    (torch.float32, 32, 16, True),
    (torch.float32, 128, 64, False),
]


@pytest.mark.parametrize("dtype,d,chunk,perkey", CASES)
def test_checkpoints_vs_oracle(dtype, d, chunk, perkey):
    lengths = [300, 1, 128, 77, 0]
    say(f"case ckpt {dtype} d={d} C={chunk} perkey={perkey} lens={lengths}")
    H = 3
    x = inputs.random_prefill(31, lengths, H=H, dk=d, dv=d, dtype=dtype, perkey=perkey,
                              chunk=chunk, with_init=True)
    n = len(lengths)
    spec = ragged_spec(chunk, lengths, first_free=n)
    n_slots = n + sum(len(e) for e in spec)
    pool0 = torch.randn(n_slots, H, d, d, generator=torch.Generator().manual_seed(5))
    pool0[:n] = x.init_states
    slots = torch.arange(n, dtype=torch.int32)
    has_init = torch.ones(n, dtype=torch.int32)

    o, pool = run_ckpt(x, pool0.clone(), slots, has_init, spec, chunk)
    o_plain, pool_plain = run_plain(x, pool0.clone(), slots, has_init, chunk)
    # the exports change nothing else: outputs and final states bit-identical
    assert torch.equal(o, o_plain)
    assert torch.equal(pool[:n], pool_plain[:n])

    bar = BAR[dtype]
    o_ref, s_ref = oracle_prefill(x)
    assert oracle.rel_err(o, o_ref) <= bar and oracle.rel_err(pool[:n], s_ref) <= bar
    n_stored = 0
    for i, entries in enumerate(spec):
        stored = expected_stored(entries, lengths[i], chunk)
        want = [p for (p, _), st in zip(entries, stored) if st]
        ref = oracle_prefix_states(x, i, want, x.init_states[i]) if want else {}
        for (p, s), st in zip(entries, stored):
            if s < 0:
                continue
            if st:
                e = oracle.rel_err(pool[s], ref[p])
                say(f"   seq {i} p={p} slot {s}: rel err {e:.2e}")
                assert e <= bar
                n_stored += 1
            else:
                assert torch.equal(pool[s], pool0[s]), (i, p, s)
    assert n_stored == (8 if chunk == 64 else 9)  # 2 C <= 77 adds one for C < 64


@pytest.mark.parametrize("dtype,perkey", [(torch.bfloat16, False), (torch.float32, True)])
def test_checkpoint_equals_prefix_prefill_bitwise(dtype, perkey):
    """The state exported at offset p is bit-identical to the final state of a plain prefill
    over the first p tokens (same chunk size, same initial state)."""
    say(f"case ckpt bitwise vs prefix prefill {dtype} perkey={perkey}")
    lengths, H, d, C = [517, 200, 64], 2, 128, 64
    x = inputs.random_prefill(32, lengths, H=H, dk=d, dv=d, dtype=dtype, perkey=perkey,
                              chunk=C, with_init=True)
    prefixes = [[64, 128, 320, 512, 517], [192, 200], [64]]
    n = len(lengths)
    spec, nxt = [], n
    for ps in prefixes:
        spec.append([(p, nxt + j) for j, p in enumerate(ps)])
        nxt += len(ps)
    pool0 = torch.zeros(nxt, H, d, d)
    pool0[:n] = x.init_states
    _, pool = run_ckpt(x, pool0, torch.arange(n, dtype=torch.int32),
                       torch.ones(n, dtype=torch.int32), spec, C)
    # all prefixes as one packed batch of their own
    cu = x.cu_seqlens
    sel, lens, init = [], [], []
    for i, ps in enumerate(prefixes):
        for p in ps:
            sel.append(torch.arange(int(cu[i]), int(cu[i]) + p))
            lens.append(p)
            init.append(x.init_states[i])
    idx = torch.cat(sel)
    y = inputs.PrefillInputs(q=x.q[idx].contiguous(), k=x.k[idx].contiguous(),
                             v=x.v[idx].contiguous(), g=x.g[idx].contiguous(),
                             beta=x.beta[idx].contiguous(),
                             cu_seqlens=torch.tensor(np.concatenate([[0], np.cumsum(lens)]),
                                                     dtype=torch.int32),
                             scale=x.scale, qk_l2norm=x.qk_l2norm, chunk=C,
                             init_states=torch.stack(init))
    m = len(lens)
    _, pref = run_plain(y, y.init_states.clone(), torch.arange(m, dtype=torch.int32),
                        torch.ones(m, dtype=torch.int32), C)
    assert torch.equal(pool[n:], pref)


def test_checkpoints_full_size_block_interval():
    """GDN prefill at full size (T=8192, H=16, d=128, chunk 64, bf16) exporting the state
    every 640 tokens (a hybrid-cache block of 640 tokens): 12 checkpoints vs the oracle."""
    say("case ckpt full size, every 640 tokens")
    x = inputs.prefill_config(0)
    T, H, d = x.total_tokens, 16, 128
    pos = list(range(640, T, 640))
    spec = [[(p, 1 + j) for j, p in enumerate(pos)]]
    pool0 = torch.zeros(1 + len(pos), H, d, d)
    o, pool = run_ckpt(x, pool0, torch.zeros(1, dtype=torch.int32), None, spec, 64)
    o_ref, s_ref = oracle_prefill(x)
    assert oracle.rel_err(o, o_ref) <= 1e-2 and oracle.rel_err(pool[:1], s_ref) <= 1e-2
    ref = oracle_prefix_states(x, 0, pos, None)
    worst = max(oracle.rel_err(pool[1 + j], ref[p]) for j, p in enumerate(pos))
    say(f"   worst checkpoint rel err {worst:.2e}")
    assert worst <= 1e-2
