"""The C-ABI library loads on a host without a GPU, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call (CPU only)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_prefill_amd import gdn
from gated_delta_rule_prefill_amd.gdn import gdn_dims_t, gdn_deltalog_pool_t

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = _declared()
    for n in ("gdn_prefill_chunked", "gdn_prefill_chunked_ckpt", "gdn_prefill_chunked_conv",
              "gdn_prefill_chunked_noalloc",
              "gdn_prefill_workspace_bytes", "gdn_decode_step", "gdn_decode_spec",
              "gdn_decode_fused",
              "gdn_decode_deltalog", "gdn_deltalog_workspace_bytes", "gdn_deltalog_reset",
              "gdn_deltalog_materialize", "gdn_conv1d_silu", "gdn_status_string",
              "gdn_last_error", "gdn_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = gdn.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert gdn.gdn_abi_version() == 1


def test_debug_library_exports_every_declared_symbol():
    """libgdn_debug.so (C-ABI layer with GDN_DEBUG_CHECKS, same kernels) is built beside
    libgdn.so and exports the same symbols."""
    path = os.path.join(os.path.dirname(gdn.LIB_PATH), "libgdn_debug.so")
    lib = ctypes.CDLL(path)
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_uses_the_c_names():
    for name in _declared():
        assert hasattr(gdn, name), name


def test_status_strings():
    assert gdn.gdn_status_string(0) == "ok"
    assert gdn.gdn_status_string(5) == "workspace too small"
    assert gdn.gdn_status_string(99) == "unknown status"


def _dims(H=4, dk=128, dv=128, dtype=1, gate=0, l2=0):
    return gdn_dims_t(H, dk, dv, dtype, gate, 0.1, l2)


FAKE = 0x7f0000000000  # aligned, never dereferenced (validation fails before any launch)


def _prefill(dims, ws_bytes=1 << 40, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, n=2, T=100, chunk=64,
             pool=FAKE, n_slots=4, slots=FAKE, has_init=None, o=FAKE, ws=FAKE)
    a.update(kw)
    lib = gdn.load()
    return lib.gdn_prefill_chunked(
        ctypes.byref(dims), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"], a["T"],
        a["chunk"], a["pool"], a["n_slots"], a["slots"], a["has_init"], a["o"], a["ws"],
        ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(ws=None), 1), (dict(slots=None), 1),
    (dict(q=FAKE + 8), 4), (dict(o=FAKE + 2), 4), (dict(has_init=FAKE + 4), 4),
    (dict(chunk=48), 3), (dict(chunk=128), 3), (dict(n=-1), 2), (dict(T=-5), 2),
    (dict(n_slots=0), 2),
])
def test_prefill_rejects_bad_arguments(kw, status):
    assert _prefill(_dims(), **kw) == status
    assert gdn.gdn_last_error() != ""


def _prefill_ckpt(dims, ws_bytes=1 << 40, n_ckpt=3, ckpt_cu=FAKE, ckpt_pos=FAKE,
                  ckpt_slots=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, n=2, T=100, chunk=64,
             pool=FAKE, n_slots=4, slots=FAKE, has_init=None, o=FAKE, ws=FAKE)
    a.update(kw)
    return gdn.load().gdn_prefill_chunked_ckpt(
        ctypes.byref(dims), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"], a["T"],
        a["chunk"], a["pool"], a["n_slots"], a["slots"], a["has_init"], ckpt_cu, ckpt_pos,
        ckpt_slots, n_ckpt, a["o"], a["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_ckpt=-1), 2), (dict(ckpt_cu=None), 1), (dict(ckpt_pos=None), 1),
    (dict(ckpt_slots=None), 1), (dict(ckpt_pos=FAKE + 4), 4), (dict(ckpt_slots=FAKE + 8), 4),
    (dict(q=None), 1), (dict(chunk=8), 3), (dict(n_slots=0), 2),
])
def test_prefill_ckpt_rejects_bad_arguments(kw, status):
    assert _prefill_ckpt(_dims(), **kw) == status
    assert gdn.gdn_last_error() != ""


def test_prefill_ckpt_zero_checkpoints_and_zero_sequences_need_no_arrays():
    # n_seqs == 0 is a no-op before any launch; with n_ckpt == 0 the arrays may be NULL
    assert _prefill_ckpt(_dims(), n=0, n_ckpt=0, ckpt_cu=None, ckpt_pos=None,
                         ckpt_slots=None, q=None, ws=None) == 0
    assert _prefill_ckpt(_dims(), n_ckpt=0, ckpt_cu=None, ckpt_pos=None, ckpt_slots=None,
                         ws=None) == 1  # the workspace check still applies


@pytest.mark.parametrize("dims,status", [
    (_dims(dk=96, dv=96), 3), (_dims(dk=64, dv=128), 3), (_dims(dtype=2), 3),
    (_dims(gate=2), 3), (_dims(H=0), 2), (_dims(l2=3), 3),
])
def test_prefill_rejects_bad_dims(dims, status):
    assert _prefill(dims) == status


def test_prefill_workspace_too_small_and_sizing():
    lib = gdn.load()
    dims = _dims(H=16, dk=128, dv=128)
    need = ctypes.c_size_t(0)
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(dims), 1, 8192, 64, ctypes.byref(need)) == 0
    # 128 chunks x 16 heads x (W, Q_in, K_g^T, M in bf16 + U in fp32, a space shared with
    # the scan's own U operands ((R - I) diag(beta) and the conv-fused call's v rows in
    # bf16, beta in fp32), + decay in fp32) + table
    per = (64 * 128 * 2 * 2 + 128 * 64 * 2 + 64 * 64 * 2
           + max(64 * 128 * 4, 64 * 64 * 2 + 64 * 4 + 64 * 128 * 2) + 128 * 4)
    # 16 (sequence, head) units leave half of the chip's CUs idle (the CU count is 256
    # without a device), so the scan runs in (at most) two segments: + L (bf16) per unit and,
    # per (sequence, head), the state at the split (fp32 and bf16) and the second segment's
    # transition and zero-state final state (fp32)
    seg = 16 * 128 * 128 * (4 + 2 + 4 + 4)
    assert need.value >= 128 * 16 * (per + 64 * 128 * 2) + seg
    assert need.value < 128 * 16 * (per + 64 * 128 * 2) + seg + 64 * 1024
    assert _prefill(dims, ws_bytes=need.value - 1, n=1, T=8192) == 5
    # 8 sequences: a larger chunk bound, (8192 + 8 x 63) / 64 = 135 chunks, and 128 units,
    # too many for two segments
    more = ctypes.c_size_t(0)
    lib.gdn_prefill_workspace_bytes(ctypes.byref(dims), 8, 8192, 64, ctypes.byref(more))
    assert 135 * 16 * per <= more.value < 135 * 16 * per + 64 * 1024
    # 4 heads: 256 / (4 x 8) = 8 segments fit, but a sequence of 128 chunks takes 128 / 20
    # = 6, so 5 segment boundaries of the four states
    four = ctypes.c_size_t(0)
    dims4 = _dims(H=4, dk=128, dv=128)
    lib.gdn_prefill_workspace_bytes(ctypes.byref(dims4), 1, 8192, 64, ctypes.byref(four))
    base4 = 128 * 4 * (per + 64 * 128 * 2) + 5 * 4 * 128 * 128 * (4 + 2 + 4 + 4)
    assert base4 <= four.value < base4 + 64 * 1024
    # d = 64, 16 heads: 4 value tiles per head, 256 / (16 x 4) = 4 segments fit and a
    # 128-chunk sequence takes them all, so 3 boundaries; + L (bf16, 64 x 64) per unit
    # (U's section holds the larger of U and the scan's own U operands with the raw-q row
    # factors; at d = 64 the latter)
    per64 = (64 * 64 * 2 * 2 + 64 * 64 * 2 + 64 * 64 * 2
             + max(64 * 64 * 4, 64 * 64 * 2 + 64 * 4 + 64 * 64 * 2 + 64 * 4) + 64 * 4)
    d64 = ctypes.c_size_t(0)
    lib.gdn_prefill_workspace_bytes(ctypes.byref(_dims(H=16, dk=64, dv=64)), 1, 8192, 64,
                                    ctypes.byref(d64))
    base64 = 128 * 16 * (per64 + 64 * 64 * 2) + 3 * 16 * 64 * 64 * (4 + 2 + 4 + 4)
    assert base64 <= d64.value < base64 + 64 * 1024
    # fp32, d = 128, 16 heads: two segments; every section in 4-byte elements (the transposed
    # state at a boundary too)
    perf = 3 * 64 * 128 * 4 + 64 * 64 * 4 + max(64 * 128 * 4, 64 * 64 * 4 + 64 * 4 + 64 * 128 * 4
                                                  + 64 * 4) + 128 * 4
    f32 = ctypes.c_size_t(0)
    lib.gdn_prefill_workspace_bytes(ctypes.byref(_dims(H=16, dtype=0)), 1, 8192, 64,
                                    ctypes.byref(f32))
    basef = 128 * 16 * (perf + 64 * 128 * 4) + 16 * 128 * 128 * (4 + 4 + 4 + 4)
    assert basef <= f32.value < basef + 64 * 1024
    # d = 32 never runs segments: the plain layout only
    d32 = ctypes.c_size_t(0)
    lib.gdn_prefill_workspace_bytes(ctypes.byref(_dims(H=1, dk=32, dv=32)), 1, 8192, 64,
                                    ctypes.byref(d32))
    per32 = (64 * 32 * 2 * 2 + 32 * 64 * 2 + 64 * 64 * 2
             + max(64 * 32 * 4, 64 * 64 * 2 + 64 * 4 + 64 * 32 * 2 + 64 * 4) + 32 * 4)
    assert 128 * per32 <= d32.value < 128 * per32 + 64 * 1024


def _prefill_noalloc(dims, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=FAKE, n=2, T=100, chunk=64,
             pool=FAKE, n_slots=4, slots=FAKE, has_init=None, o=FAKE)
    a.update(kw)
    return gdn.load().gdn_prefill_chunked_noalloc(
        ctypes.byref(dims), a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"], a["T"],
        a["chunk"], a["pool"], a["n_slots"], a["slots"], a["has_init"], a["o"], None)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m is not None
    assert int(m.group(1)) << int(m.group(2)) == gdn.GDN_NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(slots=None), 1), (dict(o=FAKE + 2), 4),
    (dict(chunk=48), 3), (dict(n=-1), 2), (dict(n_slots=0), 2),
])
def test_prefill_noalloc_rejects_bad_arguments(kw, status):
    assert _prefill_noalloc(_dims(), **kw) == status
    assert gdn.gdn_last_error() != ""


def test_prefill_noalloc_rejects_calls_beyond_its_scratch_before_any_hip_call():
    """The size check precedes every HIP call (this host has no GPU): a call whose workspace
    would exceed the per-GPU scratch returns GDN_ERR_WORKSPACE and names both sizes."""
    lib = gdn.load()
    dims = _dims(H=16, dk=128, dv=128)
    need = ctypes.c_size_t(0)
    T = 8192
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(dims), 1, T, 64, ctypes.byref(need)) == 0
    assert need.value > gdn.GDN_NOALLOC_SCRATCH_BYTES
    assert _prefill_noalloc(dims, n=1, T=T) == 5
    assert str(gdn.GDN_NOALLOC_SCRATCH_BYTES) in gdn.gdn_last_error()
    assert _prefill_noalloc(dims, n=0, q=None) == 0  # zero sequences: a no-op


def test_zero_sized_calls_are_noops_without_gpu():
    lib = gdn.load()
    d = _dims()
    assert _prefill(d, n=0, q=None, ws=None) == 0
    assert lib.gdn_decode_step(ctypes.byref(d), None, None, None, None, None, None, 1, None, 0,
                               None, None) == 0
    assert lib.gdn_conv1d_silu(None, None, None, 0, 0, 8, 4, 1, 1, None, None) == 0


def test_decode_rejects_bad_arguments():
    lib = gdn.load()
    d = _dims()
    args = [FAKE] * 6
    assert lib.gdn_decode_step(ctypes.byref(d), *args, 4, FAKE, -1, FAKE, None) == 2
    assert lib.gdn_decode_step(ctypes.byref(d), None, *args[1:], 4, FAKE, 8, FAKE, None) == 1
    assert lib.gdn_decode_step(ctypes.byref(d), *args, 0, FAKE, 8, FAKE, None) == 2
    assert lib.gdn_decode_step(None, *args, 4, FAKE, 8, FAKE, None) == 1


def _spec(dims, n_pos=4, batch=8, num_accepted=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, n_slots=64, slots=FAKE, o=FAKE)
    a.update(kw)
    return gdn.load().gdn_decode_spec(
        ctypes.byref(dims), a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["n_slots"],
        a["slots"], num_accepted, batch, n_pos, a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_pos=0), 3), (dict(n_pos=17), 3), (dict(num_accepted=None), 1),
    (dict(num_accepted=FAKE + 4), 4), (dict(slots=None), 1), (dict(q=FAKE + 2), 4),
    (dict(batch=-1), 2), (dict(n_slots=0), 2),
])
def test_decode_spec_rejects_bad_arguments(kw, status):
    assert _spec(_dims(), **kw) == status
    assert gdn.gdn_last_error() != ""


def test_decode_spec_zero_batch_is_a_noop():
    assert _spec(_dims(), batch=0, q=None, num_accepted=None) == 0


def _prefill_conv(dims, width=4, ws_bytes=1 << 40, **kw):
    a = dict(x=FAKE, w=FAKE, cs=None, g=FAKE, beta=FAKE, cu=FAKE, n=2, T=100, chunk=64,
             pool=FAKE, n_slots=4, slots=FAKE, has_init=None, o=FAKE, ws=FAKE)
    a.update(kw)
    return gdn.load().gdn_prefill_chunked_conv(
        ctypes.byref(dims), a["x"], a["w"], width, a["cs"], a["g"], a["beta"], a["cu"], a["n"],
        a["T"], a["chunk"], a["pool"], a["n_slots"], a["slots"], a["has_init"], a["o"], a["ws"],
        ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(width=1), 3), (dict(width=5), 3), (dict(x=None), 1), (dict(w=None), 1),
    (dict(x=FAKE + 2), 4), (dict(cs=FAKE + 8), 4), (dict(g=None), 1), (dict(chunk=48), 3),
    (dict(n_slots=0), 2), (dict(ws_bytes=16), 5),
])
def test_prefill_conv_rejects_bad_arguments(kw, status):
    assert _prefill_conv(_dims(gate=1), **kw) == status
    assert gdn.gdn_last_error() != ""


def test_prefill_conv_zero_sequences_is_a_noop():
    assert _prefill_conv(_dims(), n=0, x=None, ws=None) == 0


def _fused(dims, width=4, lb=-5.0, batch=8, **kw):
    a = dict(x=FAKE, w=FAKE, cs=FAKE, fb=FAKE, wl=FAKE, al=FAKE, dt=FAKE, pool=FAKE, n_slots=16,
             slots=FAKE, o=FAKE)
    a.update(kw)
    return gdn.load().gdn_decode_fused(
        ctypes.byref(dims), a["x"], a["w"], width, a["cs"], a["fb"], a["wl"], a["al"], a["dt"],
        lb, a["pool"], a["n_slots"], a["slots"], batch, a["o"], None)


@pytest.mark.parametrize("dims,kw,status", [
    (_dims(gate=0), {}, 3), (_dims(gate=1), dict(width=5), 3), (_dims(gate=1), dict(width=1), 3),
    (_dims(gate=1), dict(lb=0.0), 3), (_dims(gate=1), dict(lb=float("nan")), 3),
    (_dims(gate=1), dict(lb=float("-inf")), 3), (_dims(gate=1), dict(cs=None), 1),
    (_dims(gate=1), dict(dt=FAKE + 4), 4), (_dims(gate=1), dict(batch=-2), 2),
    (_dims(gate=1), dict(n_slots=0), 2),
])
def test_decode_fused_rejects_bad_arguments(dims, kw, status):
    assert _fused(dims, **kw) == status
    assert gdn.gdn_last_error() != ""


def test_decode_fused_zero_batch_is_a_noop():
    assert _fused(_dims(gate=1), batch=0, x=None) == 0


def test_deltalog_rejects_bad_arguments():
    lib = gdn.load()
    d = _dims()
    pool = gdn_deltalog_pool_t(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8)
    bad_m = gdn_deltalog_pool_t(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1)
    big_m = gdn_deltalog_pool_t(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 18)
    null_base = gdn_deltalog_pool_t(None, FAKE, FAKE, FAKE, FAKE, FAKE, 8)
    args = [FAKE] * 5

    def call(dims, p, batch=8):
        return lib.gdn_decode_deltalog(ctypes.byref(dims), *args, ctypes.byref(p), 4, FAKE,
                                       batch, FAKE, None, 0, None)
    assert call(d, bad_m) == 3
    assert call(d, big_m) == 3
    assert call(d, null_base) == 1
    assert call(_dims(gate=2), pool) == 3   # rejected before any launch
    ws = ctypes.c_size_t(123)
    assert lib.gdn_deltalog_workspace_bytes(ctypes.byref(d), 512, 8, ctypes.byref(ws)) == 0
    assert ws.value == 0
    assert lib.gdn_deltalog_reset(ctypes.byref(d), ctypes.byref(bad_m), 4, FAKE, 2, None) == 3


def test_conv_rejects_bad_arguments():
    lib = gdn.load()
    assert lib.gdn_conv1d_silu(FAKE, FAKE, FAKE, 1, 10, 12, 4, 1, 1, FAKE, None) == 2   # 12 % 8
    assert lib.gdn_conv1d_silu(FAKE, FAKE, FAKE, 1, 10, 40, 4, 3, 1, FAKE, None) == 2   # 40 % 24
    assert lib.gdn_conv1d_silu(FAKE, FAKE, FAKE, 1, 10, 48, 5, 1, 1, FAKE, None) == 3
    assert lib.gdn_conv1d_silu(FAKE, FAKE, FAKE, 1, 10, 48, 4, 1, 7, FAKE, None) == 3
    assert lib.gdn_conv1d_silu(FAKE + 2, FAKE, FAKE, 1, 10, 48, 4, 1, 1, FAKE, None) == 4


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(2, 1, 16)
    with pytest.raises(ValueError):
        gdn._dev(q)


def test_product_path_does_not_import_the_oracle():
    """The oracle is test infrastructure: the package and the library sources never name it."""
    pkg = os.path.join(ROOT, "gated_delta_rule_prefill_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "gdn_oracle" not in text, f
