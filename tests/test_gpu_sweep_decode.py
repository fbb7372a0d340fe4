"""Seeded sweep of decode configurations against the fp64 oracle, through the C ABI.

Each case draws element type, head dim, gate kind, L2 norm, batch, pool size and slot map
(with an inactive row, slot -1), and runs a few steps of one entry point:
  - the one-token step (a short rollout over the same slots);
  - the spec-decode verify step (n_pos tokens per request, random accepted counts; the
    round starts from the slot of column num_accepted - 1);
  - the fused KDA step (conv width 2-4, gates formed in the kernel);
  - the DeltaLog step (merge interval M = 2-6, enough steps to cross merges), against the
    dense recurrence, which it reproduces up to its bf16 key log.
Bars as elsewhere: 1e-4 (fp32 inputs), 1e-2 (bf16 inputs); DeltaLog against the dense recurrence
5e-3 (its logged keys are stored in bf16 even for fp32 inputs, so fp32 cases land at 1e-4 to
1e-3); the conv window, a copy, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, say, to_dev
from test_gpu_fused import oracle_fused, run_fused
from test_gpu_spec import oracle_round

pytestmark = pytest.mark.gpu

N_CASES = 32


def draw(seed):
    r = np.random.default_rng(5000 + seed)
    return dict(mode=["step", "spec", "fused", "deltalog"][seed % 4],
                dtype=[torch.float32, torch.bfloat16][r.integers(2)],
                d=int(r.choice([16, 32, 64, 128])), perkey=bool(r.integers(2)),
                l2=bool(r.integers(2)), H=int(r.integers(1, 4)), B=int(r.integers(1, 9)),
                P=int(r.integers(1, 6)), W=int(r.integers(2, 5)), M=int(r.integers(2, 7)),
                rng=r)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_decode_sweep_vs_oracle(seed):
    c = draw(seed)
    mode, dtype, d, perkey, l2, H, B = (c[k] for k in ("mode", "dtype", "d", "perkey", "l2",
                                                       "H", "B"))
    say(f"case decode sweep {seed}: {mode} {dtype} d={d} perkey={perkey} l2={l2} H={H} B={B} "
        f"P={c['P']} W={c['W']} M={c['M']}")
    r = c["rng"]
    bar = max(BAR[dtype], 5e-3) if mode == "deltalog" else BAR[dtype]
    scale = d ** -0.5
    n_slots = B * c["P"] + 3
    pool0 = inputs.decode_pool(6000 + seed, n_slots, H, d, d)

    if mode == "step" or mode == "deltalog":
        slots = torch.tensor([int(s) for s in r.permutation(n_slots)[:B]], dtype=torch.int32)
        if B > 1:
            slots[int(r.integers(B))] = -1
        act = [b for b in range(B) if slots[b] >= 0]
        stream = inputs.DecodeStream(7000 + seed, B, H, d, d, dtype=dtype, perkey=perkey,
                                     prenorm=not l2)
        steps = 3 if mode == "step" else 2 * c["M"] + 1
        pd = pool0.clone().to(DEV)
        sd = slots.to(DEV)
        dl = gdn.DeltaLogPool(pd, c["M"], perkey=perkey) if mode == "deltalog" else None
        S = pool0[slots[act].long()].double().numpy()
        for t in range(steps):
            q, k, v, g, b = stream.next()
            if dl is None:
                o = gdn.gdn_decode_step(*to_dev(q, k, v, g, b), pd, sd, scale=scale,
                                        qk_l2norm=l2)
            else:
                o = gdn.gdn_decode_deltalog(*to_dev(q, k, v, g, b), dl, sd, scale=scale,
                                            qk_l2norm=l2)
            torch.cuda.synchronize()
            o = o.cpu()
            o_ref, S = oracle.decode_step(q[act], k[act], v[act], g[act], b[act], S,
                                          scale=scale, l2norm=l2)
            assert oracle.rel_err(o[act], o_ref) <= bar, (seed, t)
            inactive = [b_ for b_ in range(B) if b_ not in act]
            assert all(float(o[b_].abs().max()) == 0.0 for b_ in inactive), (seed, t)
        if dl is not None:
            gdn.gdn_deltalog_materialize(dl, sd)
            torch.cuda.synchronize()
        pool = pd.cpu()
        assert oracle.rel_err(pool[slots[act].long()], S) <= bar, seed
        others = [s for s in range(n_slots) if s not in set(slots[act].tolist())]
        assert torch.equal(pool[others], pool0[others]), seed

    elif mode == "spec":
        P = c["P"]
        q, k, v, g, b = inputs.spec_round(7000 + seed, B, P, H, d, d, dtype=dtype,
                                          perkey=perkey, prenorm=not l2)
        table, acc = inputs.spec_slot_table(8000 + seed, n_slots, B, P)
        if B > 1:
            acc[int(r.integers(B))] = 0                  # an inactive request
        pd = pool0.clone().to(DEV)
        o = gdn.gdn_decode_spec(*to_dev(q, k, v, g, b), pd, table.to(DEV), acc.to(DEV),
                                scale=scale, qk_l2norm=l2)
        torch.cuda.synchronize()
        o, pool = o.cpu(), pd.cpu()
        act = [i for i in range(B) if acc[i] >= 1]
        start = torch.stack([pool0[int(table[i, int(acc[i]) - 1])] for i in act])
        o_ref, s_ref = oracle_round(q[act], k[act], v[act], g[act], b[act], start, scale, l2)
        assert oracle.rel_err(o[act], o_ref) <= bar, seed
        for j, i in enumerate(act):
            for p in range(P):
                assert oracle.rel_err(pool[int(table[i, p])], s_ref[j, p]) <= bar, (seed, i, p)

    else:  # fused KDA step: per-key gates formed in the kernel, L2 norm as drawn
        f = inputs.fused_decode_step(7000 + seed, B, n_slots, H, d, width=c["W"], dtype=dtype)
        slots = torch.tensor([int(s) for s in r.permutation(n_slots)[:B]], dtype=torch.int32)
        if B > 1:
            slots[int(r.integers(B))] = -1
        o, pool, cs = run_fused(f, pool0, slots, scale, l2=l2)
        o_ref, s_ref, act = oracle_fused(f, slots.tolist(), pool0, H, d, scale, l2=l2)
        assert oracle.rel_err(o[act], o_ref) <= bar, seed
        for j, b_ in enumerate(act):
            s = int(slots[b_])
            assert oracle.rel_err(pool[s], s_ref[j]) <= bar, (seed, b_)
            want = torch.cat([f.conv_state[s][:, 1:], f.x[b_][:, None]], 1)  # shift by one
            assert torch.equal(cs[s], want), (seed, b_)
