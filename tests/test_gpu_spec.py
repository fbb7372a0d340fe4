"""Speculative-decoding verify step on the GPU vs the fp64 oracle, through the C ABI.

The oracle of a verify round is the one-token recurrence applied n_pos times from the
state in the starting slot (column num_accepted - 1 of the request's slot row); the state
after each position is what the position's slot must hold. Bars: max|x - ref| / max|ref|
<= 1e-4 (fp32 inputs) or 1e-2 (bf16 inputs) per tensor.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, say, to_dev

pytestmark = pytest.mark.gpu


def oracle_round(q, k, v, g, b, start_states, scale, l2):
    """Chain the one-token oracle over the positions: returns o [B, P, H, dv] and the
    states after every position [B, P, H, dk, dv] (fp64)."""
    B, P = q.shape[:2]
    S = start_states.double().numpy()
    outs, states = [], []
    for j in range(P):
        o, S = oracle.decode_step(q[:, j], k[:, j], v[:, j], g[:, j], b[:, j], S, scale=scale,
                                  l2norm=l2)
        outs.append(o)
        states.append(S)
    return np.stack(outs, 1), np.stack(states, 1)


def run_spec(q, k, v, g, b, pool, table, acc, scale, l2=False):
    pd = pool.to(DEV)
    o = gdn.gdn_decode_spec(*to_dev(q, k, v, g, b), pd, table.to(DEV), acc.to(DEV),
                            scale=scale, qk_l2norm=l2)
    torch.cuda.synchronize()
    return o.cpu(), pd.cpu()


@pytest.mark.parametrize("dtype,d,perkey,l2,P", [
    (torch.float32, 16, False, False, 4), (torch.float32, 64, True, True, 3),
    (torch.float32, 128, False, False, 16), (torch.bfloat16, 32, True, False, 2),
    (torch.bfloat16, 128, False, True, 4), (torch.bfloat16, 128, True, False, 5),
    (torch.bfloat16, 128, True, True, 16),  # the largest LDS footprint the ABI accepts
])
def test_spec_vs_oracle(dtype, d, perkey, l2, P):
    """8 requests; random distinct slot rows, random num_accepted; request 6 has
    num_accepted = 0 and request 7 a starting slot of -1 (both inactive); a few positions
    of active requests keep no state (slot -1)."""
    say(f"case spec {dtype} d={d} perkey={perkey} l2={l2} P={P}")
    B, H = 8, 3
    n_slots = B * P + 5
    pool0 = inputs.decode_pool(7, n_slots, H, d, d)
    table, acc = inputs.spec_slot_table(8, n_slots, B, P)
    acc[6] = 0
    acc[7] = 1
    table[7, 0] = -1
    if P > 1:  # positions that keep no state (never a starting column)
        for r in range(4):
            j = (int(acc[r]) % P)
            if j != int(acc[r]) - 1:
                table[r, j] = -1
    q, k, v, g, b = inputs.spec_round(9, B, P, H, d, d, dtype=dtype, perkey=perkey,
                                      prenorm=not l2)
    scale = d ** -0.5
    o, after = run_spec(q, k, v, g, b, pool0, table, acc, scale, l2)

    active = [r for r in range(B) if r not in (6, 7)]
    start = torch.stack([pool0[int(table[r, int(acc[r]) - 1])] for r in active])
    o_ref, s_ref = oracle_round(q[active], k[active], v[active], g[active], b[active], start,
                                scale, l2)
    bar = BAR[dtype]
    e_o = oracle.rel_err(o[active], o_ref)
    assert np.isfinite(o.float().numpy()).all()
    assert torch.all(o[6] == 0) and torch.all(o[7] == 0)
    written = set()
    worst = 0.0
    for i, r in enumerate(active):
        for j in range(P):
            sl = int(table[r, j])
            if sl >= 0:
                worst = max(worst, oracle.rel_err(after[sl], s_ref[i, j]))
                written.add(sl)
    say(f"   rel err o={e_o:.2e} worst stored S={worst:.2e} (bar {bar:g})")
    assert e_o <= bar and worst <= bar
    for sl in range(n_slots):
        if sl not in written:
            assert torch.equal(after[sl], pool0[sl]), sl


@pytest.mark.parametrize("perkey", [False, True])
def test_single_position_equals_decode_step_bitwise(perkey):
    """n_pos = 1, num_accepted = 1 is exactly the one-token step."""
    say(f"case spec n_pos=1 vs decode_step perkey={perkey}")
    B, H, d, n_slots = 16, 4, 128, 40
    pool0 = inputs.decode_pool(10, n_slots, H, d, d)
    slots = inputs.decode_slots(11, n_slots, B)
    q, k, v, g, b = inputs.DecodeStream(12, B, H, d, d, perkey=perkey).next()
    p1 = pool0.to(DEV)
    o1 = gdn.gdn_decode_step(*to_dev(q, k, v, g, b), p1, slots.to(DEV), scale=0.1)
    o2, p2 = run_spec(q[:, None], k[:, None], v[:, None], g[:, None], b[:, None], pool0,
                      slots.view(B, 1), torch.ones(B, dtype=torch.int32), 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), o2[:, 0]) and torch.equal(p1.cpu(), p2)


def test_rollback_by_index_pages_example():
    """The pages' walk-through: slot row [41, 9, 72, 18] for inputs [x0, d1, d2, d3]; two
    drafts accepted (num_accepted = 3), so the next round starts from slot 72 = the state
    after x0, d1, d2, and rewrites the row from column 0 (slot 18's rejected snapshot is
    overwritten at position 3)."""
    say("case spec rollback example")
    H, d, P = 4, 128, 4
    n_slots = 80
    pool0 = inputs.decode_pool(13, n_slots, H, d, d)
    row = torch.tensor([[41, 9, 72, 18]], dtype=torch.int32)
    x1 = inputs.spec_round(14, 1, P, H, d, d)
    x2 = inputs.spec_round(15, 1, P, H, d, d)
    pool = pool0.to(DEV)
    rd = row.to(DEV)
    o1 = gdn.gdn_decode_spec(*to_dev(*x1), pool, rd, torch.tensor([1], dtype=torch.int32,
                                                                  device=DEV), scale=0.1)
    o2 = gdn.gdn_decode_spec(*to_dev(*x2), pool, rd, torch.tensor([3], dtype=torch.int32,
                                                                  device=DEV), scale=0.1)
    torch.cuda.synchronize()
    # oracle: prefix p (slot 41), then x0 d1 d2 of round 1, then round 2's four tokens
    o1_ref, s1 = oracle_round(*x1, pool0[41][None], 0.1, False)
    o2_ref, s2 = oracle_round(*x2, torch.from_numpy(s1[:, 2]), 0.1, False)
    assert oracle.rel_err(o1.cpu(), o1_ref) <= 1e-2
    assert oracle.rel_err(o2.cpu(), o2_ref) <= 1e-2
    after = pool.cpu()
    for j, sl in enumerate([41, 9, 72, 18]):
        assert oracle.rel_err(after[sl], s2[0, j]) <= 1e-2
    others = [s for s in range(n_slots) if s not in (41, 9, 72, 18)]
    assert torch.equal(after[others], pool0[others])


def test_spec_full_size():
    """Verify step at its full size: B = 128 requests, 4 positions (3 drafts), H = 32,
    d = 128, bf16, 1 GiB pool; every output and stored state against the oracle."""
    say("case spec full size B=128 P=4 H=32")
    B, P, H, d = 128, 4, 32, 128
    n_slots = B * P
    pool0 = inputs.decode_pool(16, n_slots, H, d, d)
    table, acc = inputs.spec_slot_table(17, n_slots, B, P)
    x = inputs.spec_round(18, B, P, H, d, d)
    o, after = run_spec(*x, pool0, table, acc, d ** -0.5)
    start = torch.stack([pool0[int(table[r, int(acc[r]) - 1])] for r in range(B)])
    o_ref, s_ref = oracle_round(*x, start, d ** -0.5, False)
    e_o = oracle.rel_err(o, o_ref)
    e_s = oracle.rel_err(after[table.long()], s_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= 1e-2 and e_s <= 1e-2
