"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run the HIP
path through the binding, and the relative-error bars."""
import sys

import torch

import oracle
from gated_delta_rule_prefill_amd import gdn

DEV = "cuda:0"

# per-tensor max relative error bars: fp32 inputs 1e-4, bf16 inputs 1e-2
BAR = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def run_prefill(x, pool=None, slots=None, has_init=None, chunk=None):
    """Run gdn_prefill_chunked on PrefillInputs x. Returns (o cpu, pool cpu)."""
    H, dk, dv = x.q.shape[1], x.q.shape[2], x.v.shape[2]
    n = x.n_seqs
    if pool is None:
        pool = torch.zeros((n, H, dk, dv), dtype=torch.float32)
        if x.init_states is not None:
            pool = x.init_states.clone().float()
    if slots is None:
        slots = torch.arange(n, dtype=torch.int32)
    if has_init is None and x.init_states is not None:
        has_init = torch.ones(n, dtype=torch.int32)
    q, k, v, g, b, cu, pd, sl, hi = to_dev(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, pool,
                                          slots, has_init)
    o = gdn.gdn_prefill_chunked(q, k, v, g, b, cu, chunk or x.chunk, pd, sl, has_init=hi,
                                scale=x.scale, qk_l2norm=x.qk_l2norm)
    torch.cuda.synchronize()
    return o.cpu(), pd.cpu()


def oracle_prefill(x, init=None, heads=None):
    """fp64 oracle on the same inputs (optionally a subset of heads)."""
    q, k, v, g, b = x.q, x.k, x.v, x.g, x.beta
    if init is None:
        init = x.init_states
    if heads is not None:
        q, k, v, g, b = (t[:, heads] for t in (q, k, v, g, b))
        if init is not None:
            init = init[:, heads]
    return oracle.recurrence(q, k, v, g, b, x.cu_seqlens, scale=x.scale, l2norm=x.qk_l2norm,
                             init_states=init)
