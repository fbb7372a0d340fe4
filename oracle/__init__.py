"""fp64 CPU oracle for the gated delta rule, DeltaLog decode and the short convolution.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library and its Python binding never do, and the oracle never
imports them. Inputs arrive as numpy / torch CPU arrays and are upcast exactly to float64.

The arithmetic lives in ``gdn_oracle.c`` (plain sequential fp64 loops, one per independent
unit, cited there section by section) and, for the chunk-wise cross-check form, in
``chunk_form.py``.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is None:
        # GDN_ORACLE_LIB selects another build of the same source (the mutation tests load
        # deliberately broken copies this way, in their own processes).
        path = os.environ.get("GDN_ORACLE_LIB", LIB)
        if path == LIB and not os.path.exists(LIB):
            build_oracle()
        lib = ctypes.CDLL(path)
        lib.gdn_oracle_recurrence.restype = ctypes.c_int
        lib.gdn_oracle_recurrence.argtypes = [
            ctypes.c_int, _ip, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _dp, _dp, _dp, _dp, _dp, ctypes.c_double, ctypes.c_int, ctypes.c_double,
            _dp, _dp, ctypes.c_int]
        lib.gdn_oracle_deltalog_step.restype = ctypes.c_int
        lib.gdn_oracle_deltalog_step.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _dp, _dp, _dp, _dp, _dp, ctypes.c_double, ctypes.c_int, ctypes.c_double,
            _dp, _dp, _dp, _dp, _dp, _ip, _dp, ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_deltalog_materialize.restype = None
        lib.gdn_oracle_deltalog_materialize.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            _dp, _dp, _dp, _dp, _dp, _ip, _dp]
        lib.gdn_oracle_conv1d_silu.restype = None
        lib.gdn_oracle_conv1d_silu.argtypes = [
            ctypes.c_int, _ip, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        _lib = lib
    return _lib


def _f64(x):
    """Exact upcast to a C-contiguous float64 numpy array (torch bf16/fp32 or numpy)."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a):
    return a.ctypes.data_as(_dp)


def _pi(a):
    return a.ctypes.data_as(_ip)


def default_threads():
    """Threads for the per-unit pool: the CPUs this process may use, capped by
    OMP_NUM_THREADS when it is set (a shared host's CPU share) and by 64."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, min(64, n))


def recurrence(q, k, v, g, beta, cu_seqlens, scale=1.0, l2norm=False, eps=1e-6,
               init_states=None, n_threads=None):
    """Sequential gated delta rule over packed varlen sequences, fp64.

    q, k: [T, H, dk]; v: [T, H, dv]; g: [T, H] (scalar gate) or [T, H, dk] (per-key gate);
    beta: [T, H]; cu_seqlens: [n+1]; init_states: [n, H, dk, dv] or None (zeros).
    Returns (o [T, H, dv], final_states [n, H, dk, dv]) as float64 numpy arrays.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    cu = _i32(cu_seqlens)
    T, H, dk = q.shape
    dv = v.shape[2]
    n = cu.shape[0] - 1
    perkey = 1 if g.ndim == 3 else 0
    assert k.shape == (T, H, dk) and v.shape[:2] == (T, H) and beta.shape == (T, H)
    assert g.shape == ((T, H, dk) if perkey else (T, H))
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    if init_states is None:
        states = np.zeros((n, H, dk, dv), dtype=np.float64)
    else:
        states = _f64(init_states).copy()
        assert states.shape == (n, H, dk, dv)
    o = np.zeros((T, H, dv), dtype=np.float64)
    nt = default_threads() if n_threads is None else n_threads
    _load().gdn_oracle_recurrence(n, _pi(cu), H, dk, dv, perkey, _p(q), _p(k), _p(v), _p(g),
                                  _p(beta), float(scale), int(bool(l2norm)), float(eps),
                                  _p(states), _p(o), int(nt))
    return o, states


def decode_step(q, k, v, g, beta, states, scale=1.0, l2norm=False, eps=1e-6, n_threads=None):
    """One recurrent step for B independent requests: q, k [B, H, dk], v [B, H, dv],
    g [B, H] or [B, H, dk], beta [B, H], states [B, H, dk, dv] (the gathered slot states).
    Returns (o [B, H, dv], new_states [B, H, dk, dv])."""
    q = _f64(q)
    B = q.shape[0]
    cu = np.arange(B + 1, dtype=np.int32)
    return recurrence(q, k, v, g, beta, cu, scale=scale, l2norm=l2norm, eps=eps,
                      init_states=states, n_threads=n_threads)


class DeltaLogState:
    """fp64 DeltaLog buffers for n independent units (DeltaLog notes §2.1 symbol table)."""

    def __init__(self, base, M, perkey=False):
        base = _f64(base)
        n, dk, dv = base.shape
        dl = dk if perkey else 1
        C = M - 1
        self.M, self.perkey, self.dk, self.dv = M, perkey, dk, dv
        self.base = base.copy()
        self.lbar = np.zeros((n, dl))
        self.klog = np.zeros((n, C, dk))
        self.ulog = np.zeros((n, C, dv))
        self.lamlog = np.zeros((n, C, dl))
        self.len = np.zeros((n,), dtype=np.int32)

    @property
    def n(self):
        return self.base.shape[0]

    def step(self, q, k, v, g, beta, scale=1.0, l2norm=False, eps=1e-6, mode=0,
             klog_bf16=True, n_threads=None):
        """One decode step on every unit; returns o [n, dv]."""
        q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
        g = g.reshape(self.n, -1)
        o = np.zeros((self.n, self.dv))
        nt = default_threads() if n_threads is None else n_threads
        rc = _load().gdn_oracle_deltalog_step(
            self.n, self.dk, self.dv, int(self.perkey), self.M, int(mode), _p(q), _p(k),
            _p(v), _p(g), _p(beta.reshape(-1).copy()), float(scale), int(bool(l2norm)),
            float(eps), _p(self.base), _p(self.lbar), _p(self.klog), _p(self.ulog),
            _p(self.lamlog), _pi(self.len), _p(o), int(bool(klog_bf16)), int(nt))
        assert rc > 0
        return o

    def materialize(self):
        """Logical state per unit (DeltaLog notes Eq. 7): [n, dk, dv]."""
        out = np.zeros_like(self.base)
        _load().gdn_oracle_deltalog_materialize(
            self.n, self.dk, self.dv, int(self.perkey), self.M, _p(self.base), _p(self.lbar),
            _p(self.klog), _p(self.ulog), _p(self.lamlog), _pi(self.len), _p(out))
        return out


def conv1d_silu(x, w, cu_seqlens):
    """Causal depthwise conv (zero history per sequence) followed by SiLU, fp64.
    x: [T, channels]; w: [channels, width]. Returns y [T, channels]."""
    x, w = _f64(x), _f64(w)
    cu = _i32(cu_seqlens)
    T, ch = x.shape
    width = w.shape[1]
    assert w.shape[0] == ch and cu[-1] == T
    y = np.zeros_like(x)
    _load().gdn_oracle_conv1d_silu(cu.shape[0] - 1, _pi(cu), ch, width, _p(x), _p(w), _p(y))
    return y


def rel_err(x, ref):
    """max|x - ref| / max|ref| over the whole tensor (the per-tensor relative error used
    for every parity bar)."""
    x = _f64(x)
    ref = _f64(ref)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref)) if x.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)
