"""The debug build (libgdn_debug.so: the C-ABI layer compiled with GDN_DEBUG_CHECKS, the same
kernels) rejects a call whose valid slot indices repeat, before any launch and without
touching memory; distinct slots, and invalid slots (outside the pool) in any number, pass
and give the release library's results bit for bit."""
import contextlib
import os

import pytest
import torch

from gated_delta_rule_prefill_amd import gdn, inputs
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(gdn.LIB_PATH), "libgdn_debug.so")


@contextlib.contextmanager
def debug_lib():
    saved = gdn._lib
    gdn._lib = None
    gdn.load(DEBUG_LIB)
    try:
        yield
    finally:
        gdn._lib = saved


def decode_inputs(B=6, H=2, d=32, n_slots=10):
    st = inputs.DecodeStream(50, B, H, d, d, dtype=torch.bfloat16)
    q, k, v, g, b = (t.to(DEV) for t in st.next())
    pool = inputs.decode_pool(51, n_slots, H, d, d).to(DEV)
    return q, k, v, g, b, pool


def expect_rejected(fn, what):
    with pytest.raises(gdn.GdnError) as e:
        fn()
    assert e.value.status == 2 and "used twice" in str(e.value), str(e.value)
    say(f"   {what}: {e.value}")


def test_decode_duplicate_slot_rejected_and_nothing_written():
    say("case debug build: decode with a repeated slot")
    q, k, v, g, b, pool = decode_inputs()
    slots = torch.tensor([3, 7, -1, 3, 9, 12], dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    pool0, o0 = pool.clone(), o.clone()
    with debug_lib():
        expect_rejected(lambda: gdn.gdn_decode_step(q, k, v, g, b, pool, slots, o=o), "decode")
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0) and torch.equal(o, o0)


def test_decode_distinct_slots_match_release():
    """Two invalid slots (-1 and 12 in a 10-slot pool) are not duplicates."""
    say("case debug build: decode with distinct slots equals the release library")
    q, k, v, g, b, pool = decode_inputs()
    slots = torch.tensor([3, 7, -1, 0, 12, -1], dtype=torch.int32, device=DEV)
    p_rel, p_dbg = pool.clone(), pool.clone()
    o_rel = gdn.gdn_decode_step(q, k, v, g, b, p_rel, slots)
    with debug_lib():
        o_dbg = gdn.gdn_decode_step(q, k, v, g, b, p_dbg, slots)
    torch.cuda.synchronize()
    assert torch.equal(o_rel, o_dbg) and torch.equal(p_rel, p_dbg)


def test_spec_and_deltalog_and_fused_duplicates_rejected():
    say("case debug build: spec table, DeltaLog and fused decode with a repeated slot")
    B, H, d, n_slots = 2, 2, 32, 12
    q, k, v, g, b, pool = decode_inputs(B * 3, H, d, n_slots)
    table = torch.tensor([[0, 1, 2], [3, 4, 1]], dtype=torch.int32, device=DEV)
    acc = torch.ones(B, dtype=torch.int32, device=DEV)
    qs, ks, vs = (t.reshape(B, 3, H, d).contiguous() for t in (q, k, v))
    gs, bs = g.reshape(B, 3, H).contiguous(), b.reshape(B, 3, H).contiguous()
    dlp = gdn.DeltaLogPool(pool.clone(), 4)
    f = inputs.fused_decode_step(52, B, n_slots, H, d, width=4)
    fb = [t.to(DEV) for t in (f.x, f.conv_w, f.conv_state, f.forget_b, f.write_logit, f.A_log,
                              f.dt_bias)]
    dup = torch.tensor([5, 5], dtype=torch.int32, device=DEV)
    with debug_lib():
        expect_rejected(lambda: gdn.gdn_decode_spec(qs, ks, vs, gs, bs, pool, table, acc),
                        "spec")
        expect_rejected(lambda: gdn.gdn_decode_deltalog(q[:B], k[:B], v[:B], g[:B], b[:B], dlp,
                                                        dup), "deltalog")
        expect_rejected(lambda: gdn.gdn_deltalog_reset(dlp, dup), "deltalog reset")
        expect_rejected(lambda: gdn.gdn_decode_fused(*fb, f.lower_bound, pool, dup), "fused")


def test_prefill_checkpoint_slot_equal_to_sequence_slot_rejected():
    say("case debug build: prefill whose checkpoint slot is a sequence's slot")
    x = inputs.random_prefill(53, [100, 40], H=2, dk=32, dv=32, chunk=32)
    q, k, v, g, b, cu = (t.to(DEV) for t in (x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens))
    pool = torch.zeros(6, 2, 32, 32, device=DEV)
    slots = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    ck_cu = torch.tensor([0, 1, 1], dtype=torch.int32, device=DEV)
    ck_pos = torch.tensor([64], dtype=torch.int32, device=DEV)
    with debug_lib():
        expect_rejected(lambda: gdn.gdn_prefill_chunked_ckpt(
            q, k, v, g, b, cu, 32, pool, slots, ck_cu, ck_pos,
            torch.tensor([1], dtype=torch.int32, device=DEV), scale=x.scale), "prefill ckpt")
        expect_rejected(lambda: gdn.gdn_prefill_chunked(
            q, k, v, g, b, cu, 32, pool, torch.tensor([4, 4], dtype=torch.int32, device=DEV),
            scale=x.scale), "prefill")
        gdn.gdn_prefill_chunked_ckpt(q, k, v, g, b, cu, 32, pool, slots, ck_cu, ck_pos,
                                     torch.tensor([5], dtype=torch.int32, device=DEV),
                                     scale=x.scale)
    torch.cuda.synchronize()
