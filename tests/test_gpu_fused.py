"""Fused KDA decode step on the GPU vs the fp64 oracle, through the C ABI.

The oracle of one step composes pinned oracle pieces: the causal convolution over each
request's window (the conv state's width - 1 inputs, oldest first, then the new input) with
SiLU (`oracle.conv1d_silu`, last position), the KDA gate formula (`oracle.gates`), and the
one-token recurrence with the per-key gate and L2 norm (`oracle.decode_step`). The conv-state
window shift is a copy and is checked bit for bit. Bars: 1e-4 (fp32 inputs), 1e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.gates import kda_forget_log, sigmoid
from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import BAR, DEV, say, to_dev

pytestmark = pytest.mark.gpu


def oracle_fused(f, slots, pool0, H, d, scale, l2=True):
    """fp64 reference of one fused step for the active rows (slot >= 0). Returns
    (o [n_active, H, d], new states [n_active, H, d, d], active row indices)."""
    act = [b for b in range(len(slots)) if slots[b] >= 0]
    W = f.conv_w.shape[1]
    # each request's window as a sequence of W inputs
    win = torch.cat([torch.cat([f.conv_state[slots[b]].T, f.x[b][None]], 0) for b in act], 0)
    cu = torch.arange(0, W * len(act) + 1, W, dtype=torch.int32)
    y = oracle.conv1d_silu(win, f.conv_w, cu)[W - 1::W]          # last position of each window
    HD = H * d
    q, k, v = (torch.from_numpy(y[:, i * HD:(i + 1) * HD]).reshape(-1, H, d) for i in range(3))
    g = kda_forget_log(f.forget_b[act].numpy(), f.dt_bias.numpy(), f.A_log.numpy(),
                       f.lower_bound)
    beta = sigmoid(f.write_logit[act].numpy())
    o, S = oracle.decode_step(q, k, v, g, beta, pool0[[slots[b] for b in act]], scale=scale,
                              l2norm=l2)
    return o, S, act


def run_fused(f, pool0, slots, scale, l2=True):
    cs = f.conv_state.clone().to(DEV)
    pool = pool0.clone().to(DEV)
    x, w, fb, wl, al, dt, sd = to_dev(f.x, f.conv_w, f.forget_b, f.write_logit, f.A_log,
                                      f.dt_bias, slots)
    o = gdn.gdn_decode_fused(x, w, cs, fb, wl, al, dt, f.lower_bound, pool, sd, scale=scale,
                             qk_l2norm=l2)
    torch.cuda.synchronize()
    return o.cpu(), pool.cpu(), cs.cpu()


@pytest.mark.parametrize("dtype,d,W,l2", [
    (torch.float32, 16, 4, True), (torch.float32, 64, 2, True), (torch.float32, 128, 3, False),
    (torch.bfloat16, 32, 4, True), (torch.bfloat16, 128, 4, True), (torch.bfloat16, 64, 3, True),
])
def test_fused_step_vs_oracle(dtype, d, W, l2):
    """8 requests over a 12-slot pool, one inactive (slot -1)."""
    say(f"case fused {dtype} d={d} W={W} l2={l2}")
    B, H, n_slots = 8, 3, 12
    f = inputs.fused_decode_step(30, B, n_slots, H, d, width=W, dtype=dtype)
    pool0 = inputs.decode_pool(31, n_slots, H, d, d)
    slots = inputs.decode_slots(32, n_slots, B)
    slots[5] = -1
    scale = d ** -0.5
    o, pool, cs = run_fused(f, pool0, slots, scale, l2)
    o_ref, S_ref, act = oracle_fused(f, slots.tolist(), pool0, H, d, scale, l2)
    bar = BAR[dtype]
    e_o = oracle.rel_err(o[act], o_ref)
    e_s = oracle.rel_err(pool[slots[act].long()], S_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e} (bar {bar:g})")
    assert e_o <= bar and e_s <= bar
    assert torch.all(o[5] == 0)
    # conv-state window: shifted by one input, exactly
    for b in act:
        s = int(slots[b])
        want = torch.cat([f.conv_state[s][:, 1:], f.x[b][:, None]], 1)
        assert torch.equal(cs[s], want), b
    used = set(int(slots[b]) for b in act)
    for s in range(n_slots):
        if s not in used:
            assert torch.equal(cs[s], f.conv_state[s]) and torch.equal(pool[s], pool0[s])


def test_fused_rollout_equals_conv_over_the_whole_stream():
    """Six fused steps from a slot whose conv state holds the three inputs before them equal
    the oracle's convolution over the nine-input stream followed by the recurrence over the
    six convolved tokens (the window is carried correctly from step to step)."""
    say("case fused rollout")
    B, H, d, W, steps = 4, 2, 64, 4, 6
    n_slots = 6
    pool0 = inputs.decode_pool(33, n_slots, H, d, d)
    slots = torch.tensor([4, 0, 2, 5], dtype=torch.int32)
    first = inputs.fused_decode_step(34, B, n_slots, H, d, width=W)
    cs = first.conv_state.clone().to(DEV)
    pool = pool0.clone().to(DEV)
    sd = slots.to(DEV)
    xs, fbs, wls, outs = [], [], [], []
    for t in range(steps):
        f = inputs.fused_decode_step(40 + t, B, n_slots, H, d, width=W)
        f.conv_w, f.A_log, f.dt_bias = first.conv_w, first.A_log, first.dt_bias
        xs.append(f.x)
        fbs.append(f.forget_b)
        wls.append(f.write_logit)
        x, w, fb, wl, al, dt = to_dev(f.x, f.conv_w, f.forget_b, f.write_logit, f.A_log,
                                      f.dt_bias)
        outs.append(gdn.gdn_decode_fused(x, w, cs, fb, wl, al, dt, -5.0, pool, sd,
                                         scale=d ** -0.5).cpu())
    torch.cuda.synchronize()
    HD = H * d
    for b in range(B):
        s = int(slots[b])
        stream = torch.cat([first.conv_state[s].T] + [x[b][None] for x in xs], 0)
        y = oracle.conv1d_silu(stream, first.conv_w, torch.tensor([0, W - 1 + steps],
                                                                  dtype=torch.int32))[W - 1:]
        q, k, v = (torch.from_numpy(y[:, i * HD:(i + 1) * HD]).reshape(steps, H, d)
                   for i in range(3))
        g = kda_forget_log(torch.stack([fb[b] for fb in fbs]).numpy(), first.dt_bias.numpy(),
                           first.A_log.numpy(), -5.0)
        beta = sigmoid(torch.stack([wl[b] for wl in wls]).numpy())
        o_ref, s_ref = oracle.recurrence(q, k, v, g, beta, torch.tensor([0, steps],
                                                                         dtype=torch.int32),
                                         scale=d ** -0.5, l2norm=True,
                                         init_states=pool0[s][None])
        got = torch.stack([o[b] for o in outs])
        assert oracle.rel_err(got, o_ref) <= 1e-2
        assert oracle.rel_err(pool.cpu()[s], s_ref[0]) <= 1e-2
        assert torch.equal(cs.cpu()[s], torch.stack([x[b] for x in xs[-(W - 1):]], 1))


def test_fused_full_size():
    """Fused KDA decode at full size: B = 128, H = 32, d = 128, width 4, bf16, 256-slot pools;
    every output and updated state against the oracle."""
    say("case fused full size B=128 H=32")
    B, H, d, n_slots = 128, 32, 128, 256
    f = inputs.fused_decode_step(35, B, n_slots, H, d)
    pool0 = inputs.decode_pool(36, n_slots, H, d, d)
    slots = inputs.decode_slots(37, n_slots, B)
    o, pool, cs = run_fused(f, pool0, slots, d ** -0.5)
    o_ref, S_ref, act = oracle_fused(f, slots.tolist(), pool0, H, d, d ** -0.5)
    e_o = oracle.rel_err(o, o_ref)
    e_s = oracle.rel_err(pool[slots.long()], S_ref)
    say(f"   rel err o={e_o:.2e} S={e_s:.2e}")
    assert e_o <= 1e-2 and e_s <= 1e-2
