"""The library's calls captured in a HIP graph (as a serving loop does) give the same results
as eager calls, replay after replay.

Every captured call is replayed several times with new inputs copied into its static
buffers, eager work and device synchronisations between the replays, and each replay is
compared with the same call run eagerly on copies (bit for bit: the same kernels run).
None of the entry points records a memory-set node.
"""
import pytest
import torch

from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _replays(n=3):
    return range(n)


def test_decode_step_graph_replays_match_eager():
    say("case graph: decode step")
    B, H, d, n_slots = 16, 4, 128, 40
    pool = inputs.decode_pool(70, n_slots, H, d, d).to(DEV)
    slots = inputs.decode_slots(71, n_slots, B).to(DEV)
    stream = inputs.DecodeStream(72, B, H, d, d)
    static = [t.to(DEV) for t in stream.next()]
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_decode_step(*static, pool.clone(), slots, scale=0.1, o=o)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn.gdn_decode_step(*static, pool, slots, scale=0.1, o=o)
    for r in _replays():
        new = [t.to(DEV) for t in stream.next()]
        for s_, n_ in zip(static, new):
            s_.copy_(n_)
        ref_pool = pool.clone()
        ref_o = gdn.gdn_decode_step(*new, ref_pool, slots, scale=0.1)   # eager on copies
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(pool, ref_pool), r


@pytest.mark.parametrize("lengths", [[300, 77, 128], [3000, 2600], [6000, 2600]])
def test_prefill_graph_replays_match_eager(lengths):
    """x 4 heads: [3000, 2600] runs the segmented scan in two segments and its combine pass,
    [6000, 2600] in four and two, with the chain pass between."""
    say(f"case graph: prefill {lengths}")
    x = inputs.random_prefill(73, lengths, H=4, dk=128, dv=128, with_init=True)
    q, k, v, g_, b, cu = to_dev(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
    n = x.n_seqs
    pool = x.init_states.clone().to(DEV)
    slots = torch.arange(n, dtype=torch.int32, device=DEV)
    hi = torch.ones(n, dtype=torch.int32, device=DEV)
    T, H, d = x.q.shape
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(H, d, d, x.q.dtype, False, n, T, 64),
                     dtype=torch.uint8, device=DEV)
    o = torch.empty((T, H, d), dtype=x.q.dtype, device=DEV)
    gdn.gdn_prefill_chunked(q, k, v, g_, b, cu, 64, pool.clone(), slots, has_init=hi,
                            scale=x.scale, o=o, workspace=ws)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        gdn.gdn_prefill_chunked(q, k, v, g_, b, cu, 64, pool, slots, has_init=hi, scale=x.scale,
                                o=o, workspace=ws)
    for r in _replays():
        y = inputs.random_prefill(74 + r, lengths, H=4, dk=128, dv=128, with_init=True)
        for s_, n_ in zip((q, k, v, g_, b), to_dev(y.q, y.k, y.v, y.g, y.beta)):
            s_.copy_(n_)
        pool.copy_(y.init_states.to(DEV))
        ref_pool = pool.clone()
        ref_o = gdn.gdn_prefill_chunked(q.clone(), k.clone(), v.clone(), g_.clone(), b.clone(),
                                        cu, 64, ref_pool, slots, has_init=hi, scale=x.scale)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(pool, ref_pool), r


def test_deltalog_cycle_graph_replays_match_eager():
    """One captured DeltaLog step replayed over more than a merge cycle (M = 4): the log
    length advances and wraps with every replay exactly as in eager steps."""
    say("case graph: DeltaLog")
    B, H, d, M = 8, 2, 64, 4
    base = inputs.decode_pool(75, B, H, d, d).to(DEV)
    slots = inputs.decode_slots(76, B, B).to(DEV)
    pool = gdn.DeltaLogPool(base.clone(), M)
    ref = gdn.DeltaLogPool(base.clone(), M)
    stream = inputs.DecodeStream(77, B, H, d, d)
    static = [t.to(DEV) for t in stream.next()]
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    warm = gdn.DeltaLogPool(base.clone(), M)
    gdn.gdn_decode_deltalog(*static, warm, slots, o=o)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        gdn.gdn_decode_deltalog(*static, pool, slots, o=o)
    for r in _replays(2 * M + 1):
        new = [t.to(DEV) for t in stream.next()]
        for s_, n_ in zip(static, new):
            s_.copy_(n_)
        ref_o = gdn.gdn_decode_deltalog(*new, ref, slots)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o), r
        for name in ("base", "lbar", "klog", "ulog", "lamlog", "len"):
            assert torch.equal(getattr(pool, name), getattr(ref, name)), (r, name)


def test_conv_prefill_graph_replays_match_eager():
    """The conv-fused prefill with a conv-state pool (prep, scan and the conv-state update in
    one capture), continuing sequences from their histories and states."""
    say("case graph: conv-fused prefill")
    lengths, H, d, W = [300, 2, 128], 2, 64, 4
    n = len(lengths)
    x = inputs.conv_prefill(75, lengths, H, d, width=W)
    X, w, g_, b, cu = to_dev(x.x, x.conv_w, x.g, x.beta, x.cu_seqlens)
    pool = x.init_states.clone().to(DEV)
    cs = x.conv_hist.clone().to(DEV)
    slots = torch.arange(n, dtype=torch.int32, device=DEV)
    hi = torch.ones(n, dtype=torch.int32, device=DEV)
    T = x.x.shape[0]
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(H, d, d, x.x.dtype, True, n, T, 64),
                     dtype=torch.uint8, device=DEV)
    o = torch.empty((T, H, d), dtype=x.x.dtype, device=DEV)
    kw = dict(has_init=hi, scale=x.scale, qk_l2norm=True)
    gdn.gdn_prefill_chunked_conv(X, w, g_, b, cu, 64, pool.clone(), slots, conv_state=cs.clone(),
                                 o=o, workspace=ws, **kw)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        gdn.gdn_prefill_chunked_conv(X, w, g_, b, cu, 64, pool, slots, conv_state=cs, o=o,
                                     workspace=ws, **kw)
    for r in _replays():
        y = inputs.conv_prefill(76 + r, lengths, H, d, width=W)
        for s_, n_ in zip((X, g_, b), to_dev(y.x, y.g, y.beta)):
            s_.copy_(n_)
        pool.copy_(y.init_states.to(DEV))
        cs.copy_(y.conv_hist.to(DEV))
        ref_pool, ref_cs = pool.clone(), cs.clone()
        ref_o = gdn.gdn_prefill_chunked_conv(X.clone(), w, g_.clone(), b.clone(), cu, 64,
                                             ref_pool, slots, conv_state=ref_cs, **kw)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(pool, ref_pool), r
        assert torch.equal(cs, ref_cs), r
