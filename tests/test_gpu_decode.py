"""Dense one-token decode over a slot-indexed state pool on the GPU vs the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,perkey,l2", [
    (torch.float32, 16, False, False), (torch.float32, 64, True, True),
    (torch.float32, 128, False, False), (torch.bfloat16, 32, True, False),
    (torch.bfloat16, 128, False, True), (torch.bfloat16, 128, True, False),
])
def test_decode_rollout_vs_oracle(dtype, d, perkey, l2):
    """20-step rollout on 12 requests with a random slot map over a 20-slot pool."""
    say(f"case decode {dtype} d={d} perkey={perkey} l2={l2}")
    B, H, n_slots, steps = 12, 3, 20, 20
    pool0 = inputs.decode_pool(1, n_slots, H, d, d)
    slots = inputs.decode_slots(2, n_slots, B)
    stream = inputs.DecodeStream(3, B, H, d, d, dtype=dtype, perkey=perkey, prenorm=not l2)
    pool = pool0.to(DEV)
    sd = slots.to(DEV)
    S = pool0[slots.long()].double().numpy()
    worst = 0.0
    for _ in range(steps):
        q, k, v, g, b = stream.next()
        o = gdn.gdn_decode_step(*to_dev(q, k, v, g, b), pool, sd, scale=d ** -0.5, qk_l2norm=l2)
        o_ref, S = oracle.decode_step(q, k, v, g, b, S, scale=d ** -0.5, l2norm=l2)
        worst = max(worst, oracle.rel_err(o.cpu(), o_ref))
    torch.cuda.synchronize()
    after = pool.cpu()
    e_s = oracle.rel_err(after[slots.long()], S)
    say(f"   worst o rel err {worst:.2e}, final S {e_s:.2e}")
    assert worst <= BAR[dtype] and e_s <= BAR[dtype]
    untouched = sorted(set(range(n_slots)) - set(slots.tolist()))
    assert torch.equal(after[untouched], pool0[untouched])


def test_inactive_rows():
    """Slots outside [0, n_slots) are padding: o rows are zero, the pool is untouched."""
    say("case decode inactive rows")
    B, H, d = 4, 2, 64
    pool0 = inputs.decode_pool(4, 3, H, d, d)
    slots = torch.tensor([2, -1, 0, 7], dtype=torch.int32)
    q, k, v, g, b = inputs.DecodeStream(5, B, H, d, d).next()
    pool = pool0.to(DEV)
    o = gdn.gdn_decode_step(*to_dev(q, k, v, g, b), pool, slots.to(DEV), scale=0.125).cpu()
    torch.cuda.synchronize()
    assert torch.all(o[1] == 0) and torch.all(o[3] == 0)
    assert torch.equal(pool.cpu()[1], pool0[1])
    o_ref, s_ref = oracle.decode_step(q[[0, 2]], k[[0, 2]], v[[0, 2]], g[[0, 2]], b[[0, 2]],
                                      pool0[[2, 0]], scale=0.125)
    assert oracle.rel_err(o[[0, 2]], o_ref) <= 1e-2
    assert oracle.rel_err(pool.cpu()[[2, 0]], s_ref) <= 1e-2


def rollout_oracle(pool0, slots, qs, ks, vs, gs, bs, scale):
    """Each request's tokens of a whole rollout as one sequence of the fp64 recurrence, from
    its slot's initial state (chaining one-token steps is exactly this recurrence). Inputs
    are per-step lists of [B, ...] tensors; returns (o [steps, B, H, d], final [B, H, d, d])."""
    steps, B = len(qs), qs[0].shape[0]
    pack = lambda ts: torch.stack(ts, 1).reshape(B * steps, *ts[0].shape[1:])
    cu = torch.arange(0, B * steps + 1, steps, dtype=torch.int32)
    o, S = oracle.recurrence(pack(qs), pack(ks), pack(vs), pack(gs), pack(bs), cu, scale=scale,
                             init_states=pool0[slots.long()])
    return np.ascontiguousarray(o.reshape(B, steps, *o.shape[1:]).swapaxes(0, 1)), S


def test_decode_config_rollout_full():
    """GDN batched decode step at full size: B=128, H=32, d=128, 256-slot fp32 pool with a
    random slot map, bf16 q/k/v, 128-step rollout. Every output of every (request, head) at
    every step and every final state are compared with the oracle; the 128 unused slots are
    canaries and must stay bit-identical."""
    say("case decode B=128 H=32 128 steps, every unit")
    B, H, d, n_slots, steps = 128, 32, 128, 256, 128
    pool0 = inputs.decode_pool(1, n_slots, H, d, d)
    slots = inputs.decode_slots(0, n_slots, B)
    stream = inputs.DecodeStream(0, B, H, d, d)
    pool = pool0.to(DEV)
    sd = slots.to(DEV)
    ins, outs = [], []
    for step in range(steps):
        x = stream.next()
        ins.append(x)
        outs.append(gdn.gdn_decode_step(*to_dev(*x), pool, sd, scale=d ** -0.5))
    torch.cuda.synchronize()
    o = torch.stack(outs).cpu()
    after = pool.cpu()
    say("   GPU rollout done; oracle over all 4096 units")
    o_ref, S = rollout_oracle(pool0, slots, *zip(*ins), scale=d ** -0.5)
    per_step = [oracle.rel_err(o[t], o_ref[t]) for t in range(steps)]
    e_o = oracle.rel_err(o, o_ref)
    e_s = oracle.rel_err(after[slots.long()], S)
    say(f"   o rel err {e_o:.2e} (worst step {max(per_step):.2e}), final S {e_s:.2e}")
    assert max(per_step) <= 1e-2 and e_o <= 1e-2 and e_s <= 1e-2
    canary = sorted(set(range(n_slots)) - set(slots.tolist()))
    assert torch.equal(after[canary], pool0[canary])
