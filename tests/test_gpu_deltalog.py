"""DeltaLog decode (dense base + append log, merge every M steps) on the GPU, against the
oracle's DeltaLog bookkeeping, the oracle's dense recurrence and the GPU dense decode."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_prefill_amd import gdn, inputs
from test_gpu_decode import rollout_oracle
from gpu_util import DEV, say, to_dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_scalar_worked_example_embedded():
    """DeltaLog notes §2.3 teaching example embedded at d = 16: k = e1, beta = 1,
    alpha = 1/2, S0[0,0] = 10 and v chosen so the corrected updates are 2, 3, 4
    (v_t = S_{t-1}[0,0]/2 + increment); M = 3 -> logical 7, 6.5, 7.25; base 10, 10, 7.25."""
    say("case deltalog worked example")
    ex = json.load(open(os.path.join(GOLDEN, "deltalog_scalar_example.json")))
    d = 16
    base = torch.zeros((1, 1, d, d), device=DEV)
    base[0, 0, 0, 0] = ex["S0"]
    pool = gdn.DeltaLogPool(base, M=ex["M"])
    slots = torch.zeros(1, dtype=torch.int32, device=DEV)
    e1 = torch.zeros((1, 1, d), device=DEV)
    e1[0, 0, 0] = 1.0
    logical = ex["S0"]
    for t, inc in enumerate(ex["increments"]):
        v = torch.zeros((1, 1, d), device=DEV)
        v[0, 0, 0] = logical * ex["decay"] + inc       # residual after decay = increment
        g = torch.full((1, 1), math.log(ex["decay"]), device=DEV)
        o = gdn.gdn_decode_deltalog(e1, e1, v, g, torch.ones((1, 1), device=DEV), pool, slots)
        torch.cuda.synchronize()
        logical = ex["logical_state"][t]
        assert abs(o[0, 0, 0].item() - logical) < 1e-5
        assert abs(pool.base[0, 0, 0, 0].item() - ex["base"][t]) < 1e-5
    assert pool.len[0, 0].item() == 0
    assert abs(pool.ulog[0, 0, 0, 0].item() - 2.0) < 1e-5
    assert abs(pool.ulog[0, 0, 1, 0].item() - 3.0) < 1e-5


@pytest.mark.parametrize("dtype,d,M,l2,perkey", [
    (torch.float32, 16, 2, False, False), (torch.float32, 64, 3, False, False),
    (torch.bfloat16, 128, 8, False, False), (torch.bfloat16, 32, 17, True, False),
    (torch.float32, 16, 3, False, True), (torch.float32, 128, 4, True, True),
    (torch.bfloat16, 128, 4, False, True), (torch.bfloat16, 64, 17, False, True),
])
def test_deltalog_vs_oracle_bookkeeping(dtype, d, M, l2, perkey):
    """Step by step against the oracle's DeltaLog (same bf16 key log), and against the
    oracle's dense recurrence; includes a batch where slots sit at different log lengths.
    perkey: KDA-style per-key-channel decay (lbar and Lambda d_k wide)."""
    say(f"case deltalog {dtype} d={d} M={M} l2={l2} perkey={perkey}")
    B, H, n_slots, steps = 6, 2, 9, 2 * M + 3
    base0 = inputs.decode_pool(6, n_slots, H, d, d)
    slots = inputs.decode_slots(7, n_slots, B)
    stream = inputs.DecodeStream(8, B, H, d, d, dtype=dtype, perkey=perkey, prenorm=not l2)
    pool = gdn.DeltaLogPool(base0.to(DEV), M, perkey=perkey)
    # stagger the log lengths: advance half the requests by some steps first
    sl = slots.long()
    ref = oracle.DeltaLogState(base0[sl].reshape(B * H, d, d).double().numpy(), M,
                               perkey=perkey)
    dense = base0[sl].double().numpy()
    sd = slots.to(DEV)
    worst_o = worst_dense = 0.0
    for step in range(steps):
        q, k, v, g, b = stream.next()
        active = torch.arange(B) if step % 3 else torch.arange(B // 2)
        sub = slots.clone()
        sub[[i for i in range(B) if i not in active.tolist()]] = -1   # inactive rows
        o = gdn.gdn_decode_deltalog(*to_dev(q, k, v, g, b), pool, sub.to(DEV), scale=0.2,
                                    qk_l2norm=l2).cpu()
        # oracle on the active rows only
        idx = torch.tensor([i * H + h for i in active.tolist() for h in range(H)])
        full_o = np.zeros((B * H, d))
        sub_state = oracle.DeltaLogState(np.zeros((len(idx), d, d)), M, perkey=perkey)
        for name in ("base", "lbar", "klog", "ulog", "lamlog", "len"):
            getattr(sub_state, name)[:] = getattr(ref, name)[idx.numpy()]
        f = lambda t: t.reshape(B * H, -1)[idx]
        o_ref = sub_state.step(f(q), f(k), f(v), f(g), f(b).reshape(-1), scale=0.2, l2norm=l2)
        for name in ("base", "lbar", "klog", "ulog", "lamlog", "len"):
            getattr(ref, name)[idx.numpy()] = getattr(sub_state, name)
        full_o[idx.numpy()] = o_ref
        od, sd_new = oracle.decode_step(q[active], k[active], v[active], g[active], b[active],
                                        dense[active.numpy()], scale=0.2, l2norm=l2)
        dense[active.numpy()] = sd_new
        got = o.reshape(B * H, d)[idx]
        worst_o = max(worst_o, oracle.rel_err(got, o_ref))
        worst_dense = max(worst_dense, oracle.rel_err(got, od.reshape(-1, d)))
        assert torch.all(o[[i for i in range(B) if i not in active.tolist()]] == 0)
    torch.cuda.synchronize()
    say(f"   worst o vs oracle-DeltaLog {worst_o:.2e}, vs oracle-dense {worst_dense:.2e}")
    bar = 1e-4 if dtype == torch.float32 else 1e-2
    assert worst_o <= bar
    assert worst_dense <= 5e-3
    assert np.array_equal(pool.len.cpu()[sl].reshape(-1).numpy(), ref.len)
    # materialize: base then equals the dense state
    gdn.gdn_deltalog_materialize(pool, sd)
    torch.cuda.synchronize()
    assert torch.all(pool.len.cpu()[sl] == 0)
    assert oracle.rel_err(pool.base.cpu()[sl], dense) <= 5e-3
    assert oracle.rel_err(pool.base.cpu()[sl].reshape(B * H, d, d), ref.materialize()) <= bar


@pytest.mark.parametrize("perkey", [False, True])
def test_reset_clears_log_keeps_base(perkey):
    say(f"case deltalog reset perkey={perkey}")
    d, H = 32, 2
    base0 = inputs.decode_pool(9, 4, H, d, d).to(DEV)
    pool = gdn.DeltaLogPool(base0.clone(), 4, perkey=perkey)
    slots = torch.tensor([1, 3], dtype=torch.int32, device=DEV)
    q, k, v, g, b = inputs.DecodeStream(10, 2, H, d, d, perkey=perkey).next()
    gdn.gdn_decode_deltalog(*to_dev(q, k, v, g, b), pool, slots)
    gdn.gdn_deltalog_reset(pool, slots)
    torch.cuda.synchronize()
    assert torch.all(pool.len == 0) and torch.all(pool.lbar == 0)
    assert torch.equal(pool.base, base0)


def test_deltalog_gate_kind_must_match_pool():
    d, H = 32, 2
    pool = gdn.DeltaLogPool(torch.zeros((2, H, d, d), device=DEV), 4, perkey=True)
    q, k, v, g, b = to_dev(*inputs.DecodeStream(11, 1, H, d, d).next())
    with pytest.raises(ValueError):
        gdn.gdn_decode_deltalog(q, k, v, g, b, pool, torch.zeros(1, dtype=torch.int32,
                                                                  device=DEV))


def _full_rollout(B, H, d, M, steps, perkey, seeds):
    """DeltaLog and dense decode on identical inputs over a whole rollout on the GPU; every
    DeltaLog output of every (request, head) at every step against the exact dense recurrence
    (oracle, each request's tokens as one sequence), the materialised DeltaLog state against
    the oracle's final states and the GPU dense state."""
    base0 = inputs.decode_pool(seeds[0], B, H, d, d)
    slots = inputs.decode_slots(seeds[1], B, B)
    dense = base0.to(DEV)
    pool = gdn.DeltaLogPool(base0.to(DEV), M, perkey=perkey)
    sd = slots.to(DEV)
    stream = inputs.DecodeStream(seeds[2], B, H, d, d, perkey=perkey)
    ins, o_log, worst_vs_dense = [], [], 0.0
    for step in range(steps):
        x = stream.next()
        ins.append(x)
        q, k, v, g, b = to_dev(*x)
        od = gdn.gdn_decode_step(q, k, v, g, b, dense, sd, scale=d ** -0.5)
        ol = gdn.gdn_decode_deltalog(q, k, v, g, b, pool, sd, scale=d ** -0.5)
        worst_vs_dense = max(worst_vs_dense, oracle.rel_err(ol.float().cpu(), od.float().cpu()))
        o_log.append(ol.cpu())
    gdn.gdn_deltalog_materialize(pool, sd)
    torch.cuda.synchronize()
    say(f"   GPU rollout done; oracle over all {B * H} units")
    o_ref, S = rollout_oracle(base0, slots, *zip(*ins), scale=d ** -0.5)
    o_log = torch.stack(o_log)
    per_step = [oracle.rel_err(o_log[t], o_ref[t]) for t in range(steps)]
    e_s = oracle.rel_err(pool.base.cpu()[slots.long()], S)
    e_sd = oracle.rel_err(pool.base.cpu(), dense.cpu())
    say(f"   DeltaLog o vs oracle: worst step {max(per_step):.2e}; materialised state vs "
        f"oracle {e_s:.2e}, vs GPU dense {e_sd:.2e}; o DeltaLog vs dense {worst_vs_dense:.2e}")
    assert max(per_step) <= 5e-3 and e_s <= 5e-3 and e_sd <= 5e-3
    assert worst_vs_dense <= 1e-2


def test_deltalog_config_vs_dense_full_size():
    """DeltaLog decode vs dense decode at full size: B=512, H=32, d=128, fp32 state (1 GiB
    per layer), M=8 (log capacity 7), 128-step rollout (16 merge cycles), identical inputs.
    5e-3 bar ([DeltaLog] §4.5, rollout error) for every DeltaLog output and the materialised
    state against the exact dense recurrence; DeltaLog and dense GPU outputs are both rounded
    to bf16, so they are compared with each other at the bf16 bar (one bf16 ulp apart at
    most, up to 2^-7 of an element)."""
    say("case deltalog B=512 vs dense, 128 steps, every unit")
    _full_rollout(512, 32, 128, 8, 128, False, (1, 0, 0))


def test_kda_deltalog_vs_dense_full_size():
    """KDA DeltaLog (per-key decay, M = 4 as the notes use for KDA) vs per-key dense decode at
    full size: B = 512, H = 32, d = 128, 128-step rollout (43 merge cycles), identical inputs,
    with the bars of the scalar case."""
    say("case KDA deltalog B=512 vs dense, 128 steps, every unit")
    _full_rollout(512, 32, 128, 4, 128, True, (2, 3, 4))
