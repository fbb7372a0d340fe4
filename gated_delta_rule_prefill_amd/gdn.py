"""Thin ctypes binding of libgdn.so (include/gdn.h). Argument marshalling only: every step
of the computation runs in the library's HIP kernels; there is no CPU fallback, and a
missing library raises.

Functions carry the C names. Tensors are torch CUDA (HIP) tensors; the HIP stream is the
current torch stream unless one is given.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB names another build of the same library (for instance one whose host code carries
# sanitizers); by default the in-tree libgdn.so
LIB_PATH = os.environ.get("GDN_LIB") or os.path.join(HERE, "libgdn.so")

GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
# include/gdn.h GDN_NOALLOC_SCRATCH_BYTES: the allocation-free prefill's per-GPU workspace
GDN_NOALLOC_SCRATCH_BYTES = 128 << 20
GDN_GATE_SCALAR, GDN_GATE_PER_KEY = 0, 1


class GdnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status} ({msg})")
        self.status = status


class gdn_dims_t(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("gate", ctypes.c_int32), ("scale", ctypes.c_float),
                ("qk_l2norm", ctypes.c_int32)]


class gdn_deltalog_pool_t(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("lbar", ctypes.c_void_p), ("klog", ctypes.c_void_p),
                ("ulog", ctypes.c_void_p), ("lamlog", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("M", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_DIMS = ctypes.POINTER(gdn_dims_t)
_POOL = ctypes.POINTER(gdn_deltalog_pool_t)

_SIGS = {
    "gdn_prefill_workspace_bytes": [_DIMS, _I, _I, _I, ctypes.POINTER(_SZ)],
    "gdn_prefill_chunked": [_DIMS, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P, _P, _P, _P,
                            _SZ, _P],
    "gdn_prefill_chunked_ckpt": [_DIMS, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P, _P,
                                 _P, _P, _P, _I, _P, _P, _SZ, _P],
    "gdn_prefill_chunked_conv": [_DIMS, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P,
                                 _P, _P, _P, _SZ, _P],
    "gdn_prefill_chunked_noalloc": [_DIMS, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _I, _P,
                                    _P, _P, _P],
    "gdn_decode_step": [_DIMS, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P],
    "gdn_decode_spec": [_DIMS, _P, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _P, _P],
    "gdn_decode_fused": [_DIMS, _P, _P, _I, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I, _P, _I,
                         _P, _P],
    "gdn_deltalog_workspace_bytes": [_DIMS, _I, _I, ctypes.POINTER(_SZ)],
    "gdn_decode_deltalog": [_DIMS, _P, _P, _P, _P, _P, _POOL, _I, _P, _I, _P, _P, _SZ, _P],
    "gdn_deltalog_reset": [_DIMS, _POOL, _I, _P, _I, _P],
    "gdn_deltalog_materialize": [_DIMS, _POOL, _I, _P, _I, _P],
    "gdn_conv1d_silu": [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P],
    "gdn_status_string": [ctypes.c_int],
    "gdn_last_error": [],
    "gdn_abi_version": [],
}


def load(path: str = LIB_PATH):
    """Load libgdn.so (built in-tree by build_lib.py). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} not found: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(path)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def lib():
    return load()


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


def gdn_abi_version() -> int:
    return int(lib().gdn_abi_version())


def _check(fn, status):
    if status != 0:
        raise GdnError(fn, status, gdn_last_error() or gdn_status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    raise TypeError(f"q/k/v must be fp32 or bf16, got {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def make_dims(H, dk, dv, dtype_code, perkey, scale, qk_l2norm):
    return gdn_dims_t(int(H), int(dk), int(dv), int(dtype_code),
                      GDN_GATE_PER_KEY if perkey else GDN_GATE_SCALAR, float(scale),
                      1 if qk_l2norm else 0)


# ---------------------------------------------------------------------------- prefill
def gdn_prefill_workspace_bytes(H, dk, dv, dtype, perkey, n_seqs, total_tokens, chunk):
    dims = make_dims(H, dk, dv, dtype if isinstance(dtype, int) else
                     (GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32),
                     perkey, 1.0, False)
    out = _SZ(0)
    _check("gdn_prefill_workspace_bytes",
           lib().gdn_prefill_workspace_bytes(ctypes.byref(dims), int(n_seqs), int(total_tokens),
                                             int(chunk), ctypes.byref(out)))
    return int(out.value)


def gdn_prefill_chunked(q, k, v, g, beta, cu_seqlens, chunk, state_pool, slots, has_init=None,
                        scale=1.0, qk_l2norm=False, o=None, workspace=None, stream=None):
    """Chunked prefill. q, k [T,H,dk]; v [T,H,dv]; g [T,H] or [T,H,dk] fp32; beta [T,H] fp32;
    cu_seqlens [n+1] int32; state_pool [slots,H,dk,dv] fp32 (updated in place);
    slots [n] int32; has_init [n] int32 or None. Returns o [T,H,dv]."""
    T, H, dk = q.shape
    dv = v.shape[2]
    n = cu_seqlens.numel() - 1
    perkey = g.dim() == 3
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    need = gdn_prefill_workspace_bytes(H, dk, dv, _dtype_code(q), perkey, n, T, chunk)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k, v, g, beta, cu_seqlens, state_pool, slots, has_init, o, workspace)
    dims = make_dims(H, dk, dv, _dtype_code(q), perkey, scale, qk_l2norm)
    _check("gdn_prefill_chunked", lib().gdn_prefill_chunked(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
        int(n), int(T), int(chunk), _ptr(state_pool), int(state_pool.shape[0]), _ptr(slots),
        _ptr(has_init), _ptr(o), _ptr(workspace), int(workspace.numel()), _stream(stream)))
    return o


def gdn_prefill_chunked_noalloc(q, k, v, g, beta, cu_seqlens, chunk, state_pool, slots,
                                has_init=None, scale=1.0, qk_l2norm=False, o=None,
                                stream=None):
    """gdn_prefill_chunked without a workspace: the library's per-GPU scratch array serves
    as one (at most GDN_NOALLOC_SCRATCH_BYTES). Nothing is allocated when `o` is given.
    Arguments as gdn_prefill_chunked. Returns o."""
    T, H, dk = q.shape
    dv = v.shape[2]
    n = cu_seqlens.numel() - 1
    perkey = g.dim() == 3
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    _dev(q, k, v, g, beta, cu_seqlens, state_pool, slots, has_init, o)
    dims = make_dims(H, dk, dv, _dtype_code(q), perkey, scale, qk_l2norm)
    _check("gdn_prefill_chunked_noalloc", lib().gdn_prefill_chunked_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
        int(n), int(T), int(chunk), _ptr(state_pool), int(state_pool.shape[0]), _ptr(slots),
        _ptr(has_init), _ptr(o), _stream(stream)))
    return o


def gdn_prefill_chunked_ckpt(q, k, v, g, beta, cu_seqlens, chunk, state_pool, slots,
                             ckpt_cu, ckpt_pos, ckpt_slots, has_init=None, scale=1.0,
                             qk_l2norm=False, o=None, workspace=None, stream=None):
    """Chunked prefill that also writes the state after ckpt_pos[i] tokens of its sequence
    into pool slot ckpt_slots[i]; the entries of sequence n are ckpt_cu[n]:ckpt_cu[n+1]
    (all three int32 device tensors). Other arguments as gdn_prefill_chunked. Returns o."""
    T, H, dk = q.shape
    dv = v.shape[2]
    n = cu_seqlens.numel() - 1
    perkey = g.dim() == 3
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    need = gdn_prefill_workspace_bytes(H, dk, dv, _dtype_code(q), perkey, n, T, chunk)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(q, k, v, g, beta, cu_seqlens, state_pool, slots, has_init, ckpt_cu, ckpt_pos,
         ckpt_slots, o, workspace)
    dims = make_dims(H, dk, dv, _dtype_code(q), perkey, scale, qk_l2norm)
    _check("gdn_prefill_chunked_ckpt", lib().gdn_prefill_chunked_ckpt(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
        int(n), int(T), int(chunk), _ptr(state_pool), int(state_pool.shape[0]), _ptr(slots),
        _ptr(has_init), _ptr(ckpt_cu), _ptr(ckpt_pos), _ptr(ckpt_slots), int(ckpt_pos.numel()),
        _ptr(o), _ptr(workspace), int(workspace.numel()), _stream(stream)))
    return o


def gdn_prefill_chunked_conv(x, conv_w, g, beta, cu_seqlens, chunk, state_pool, slots,
                             conv_state=None, has_init=None, scale=1.0, qk_l2norm=False,
                             o=None, workspace=None, stream=None):
    """Chunked prefill with the short convolution and SiLU fused into its loads.
    x [T, 3 H d] raw q|k|v projection; conv_w [3 H d, W] fp32; conv_state [slots, 3 H d, W-1]
    (x's dtype) or None: read as the history of sequences with has_init and overwritten with
    each sequence's last W-1 rows. g [T,H] or [T,H,d]; other arguments as
    gdn_prefill_chunked. Returns o [T, H, d]."""
    T = x.shape[0]
    H = beta.shape[1]
    d = x.shape[1] // (3 * H)
    W = conv_w.shape[1]
    n = cu_seqlens.numel() - 1
    perkey = g.dim() == 3
    if o is None:
        o = torch.empty((T, H, d), dtype=x.dtype, device=x.device)
    need = gdn_prefill_workspace_bytes(H, d, d, _dtype_code(x), perkey, n, T, chunk)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(x, conv_w, conv_state, g, beta, cu_seqlens, state_pool, slots, has_init, o, workspace)
    dims = make_dims(H, d, d, _dtype_code(x), perkey, scale, qk_l2norm)
    _check("gdn_prefill_chunked_conv", lib().gdn_prefill_chunked_conv(
        ctypes.byref(dims), _ptr(x), _ptr(conv_w), int(W), _ptr(conv_state), _ptr(g),
        _ptr(beta), _ptr(cu_seqlens), int(n), int(T), int(chunk), _ptr(state_pool),
        int(state_pool.shape[0]), _ptr(slots), _ptr(has_init), _ptr(o), _ptr(workspace),
        int(workspace.numel()), _stream(stream)))
    return o


# ----------------------------------------------------------------------------- decode
def gdn_decode_step(q, k, v, g, beta, state_pool, slots, scale=1.0, qk_l2norm=False, o=None,
                    stream=None):
    """One decode step. q, k [B,H,dk]; v [B,H,dv]; g [B,H] or [B,H,dk]; beta [B,H];
    state_pool [slots,H,dk,dv] fp32 updated in place; slots [B] int32. Returns o."""
    B, H, dk = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _dev(q, k, v, g, beta, state_pool, slots, o)
    dims = make_dims(H, dk, dv, _dtype_code(q), g.dim() == 3, scale, qk_l2norm)
    _check("gdn_decode_step", lib().gdn_decode_step(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
        int(state_pool.shape[0]), _ptr(slots), int(B), _ptr(o), _stream(stream)))
    return o


# --------------------------------------------------------------------------- DeltaLog
def gdn_decode_spec(q, k, v, g, beta, state_pool, spec_slots, num_accepted, scale=1.0,
                    qk_l2norm=False, o=None, stream=None):
    """Speculative-decoding verify step. q, k [B,P,H,dk]; v [B,P,H,dv]; g [B,P,H] or
    [B,P,H,dk] fp32; beta [B,P,H] fp32; state_pool [slots,H,dk,dv] fp32; spec_slots [B,P]
    int32; num_accepted [B] int32. Returns o [B,P,H,dv]."""
    B, P, H, dk = q.shape
    dv = v.shape[3]
    perkey = g.dim() == 4
    if o is None:
        o = torch.empty((B, P, H, dv), dtype=q.dtype, device=q.device)
    _dev(q, k, v, g, beta, state_pool, spec_slots, num_accepted, o)
    dims = make_dims(H, dk, dv, _dtype_code(q), perkey, scale, qk_l2norm)
    _check("gdn_decode_spec", lib().gdn_decode_spec(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
        int(state_pool.shape[0]), _ptr(spec_slots), _ptr(num_accepted), int(B), int(P), _ptr(o),
        _stream(stream)))
    return o


def gdn_decode_fused(x, conv_w, conv_state, forget_b, write_logit, A_log, dt_bias, lower_bound,
                     state_pool, slots, scale=1.0, qk_l2norm=True, o=None, stream=None):
    """Fused KDA decode step. x [B, 3 H d] (q|k|v before the convolution); conv_w [3 H d, W]
    fp32; conv_state [slots, 3 H d, W-1] (x's dtype, updated in place); forget_b [B, H, d],
    write_logit [B, H], A_log [H], dt_bias [H, d] fp32; state_pool [slots, H, d, d] fp32;
    slots [B] int32. Returns o [B, H, d]."""
    B, H, dk = forget_b.shape
    W = conv_w.shape[1]
    if o is None:
        o = torch.empty((B, H, dk), dtype=x.dtype, device=x.device)
    _dev(x, conv_w, conv_state, forget_b, write_logit, A_log, dt_bias, state_pool, slots, o)
    dims = make_dims(H, dk, dk, _dtype_code(x), True, scale, qk_l2norm)
    _check("gdn_decode_fused", lib().gdn_decode_fused(
        ctypes.byref(dims), _ptr(x), _ptr(conv_w), int(W), _ptr(conv_state), _ptr(forget_b),
        _ptr(write_logit), _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(state_pool),
        int(state_pool.shape[0]), _ptr(slots), int(B), _ptr(o), _stream(stream)))
    return o


class DeltaLogPool:
    """Device buffers of a DeltaLog state pool (layouts of gdn_deltalog_pool_t)."""

    def __init__(self, base, M, perkey=False):
        n_slots, H, dk, dv = base.shape
        C = M - 1
        dl = (dk,) if perkey else ()
        dev = base.device
        self.base = base
        self.M = int(M)
        self.perkey = bool(perkey)
        self.lbar = torch.zeros((n_slots, H, *dl), dtype=torch.float32, device=dev)
        self.klog = torch.zeros((n_slots, H, C, dk), dtype=torch.int16, device=dev)
        self.ulog = torch.zeros((n_slots, H, C, dv), dtype=torch.float32, device=dev)
        self.lamlog = torch.zeros((n_slots, H, C, *dl), dtype=torch.float32, device=dev)
        self.len = torch.zeros((n_slots, H), dtype=torch.int32, device=dev)

    @property
    def n_slots(self):
        return int(self.base.shape[0])

    def struct(self):
        _dev(self.base, self.lbar, self.klog, self.ulog, self.lamlog, self.len)
        return gdn_deltalog_pool_t(self.base.data_ptr(), self.lbar.data_ptr(),
                                   self.klog.data_ptr(), self.ulog.data_ptr(),
                                   self.lamlog.data_ptr(), self.len.data_ptr(), self.M)


def gdn_deltalog_workspace_bytes(H, dk, dv, dtype, batch, M):
    dims = make_dims(H, dk, dv, dtype, False, 1.0, False)
    out = _SZ(0)
    _check("gdn_deltalog_workspace_bytes", lib().gdn_deltalog_workspace_bytes(
        ctypes.byref(dims), int(batch), int(M), ctypes.byref(out)))
    return int(out.value)


def gdn_decode_deltalog(q, k, v, g, beta, pool: DeltaLogPool, slots, scale=1.0,
                        qk_l2norm=False, o=None, stream=None):
    B, H, dk = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _dev(q, k, v, g, beta, slots, o)
    if (g.dim() == 3) != pool.perkey:
        raise ValueError("gate kind does not match the DeltaLog pool layout")
    dims = make_dims(H, dk, dv, _dtype_code(q), g.dim() == 3, scale, qk_l2norm)
    ps = pool.struct()
    _check("gdn_decode_deltalog", lib().gdn_decode_deltalog(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), ctypes.byref(ps),
        pool.n_slots, _ptr(slots), int(B), _ptr(o), None, 0, _stream(stream)))
    return o


def _dl_maint(name, pool, slots, stream):
    n_slots, H, dk, dv = pool.base.shape
    dims = make_dims(H, dk, dv, GDN_DTYPE_F32, pool.perkey, 1.0, False)
    _dev(slots)
    ps = pool.struct()
    _check(name, getattr(lib(), name)(ctypes.byref(dims), ctypes.byref(ps), pool.n_slots,
                                      _ptr(slots), int(slots.numel()), _stream(stream)))


def gdn_deltalog_reset(pool: DeltaLogPool, slots, stream=None):
    _dl_maint("gdn_deltalog_reset", pool, slots, stream)


def gdn_deltalog_materialize(pool: DeltaLogPool, slots, stream=None):
    _dl_maint("gdn_deltalog_materialize", pool, slots, stream)


# ----------------------------------------------------------------------------- conv1d
def gdn_conv1d_silu(x, w, cu_seqlens, planes=1, y=None, stream=None):
    """x [T, channels]; w [channels, width] fp32. Returns y [planes, T, channels/planes]."""
    T, ch = x.shape
    if y is None:
        y = torch.empty((planes, T, ch // planes), dtype=x.dtype, device=x.device)
    _dev(x, w, cu_seqlens, y)
    _check("gdn_conv1d_silu", lib().gdn_conv1d_silu(
        _ptr(x), _ptr(w), _ptr(cu_seqlens), int(cu_seqlens.numel() - 1), int(T), int(ch),
        int(w.shape[1]), int(planes), _dtype_code(x), _ptr(y), _stream(stream)))
    return y
