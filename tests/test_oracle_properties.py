"""Property tests of the fp64 oracle (CPU only), with hypothesis drawing shapes, ragged
lengths, chunk sizes and gate values. Each property is a fact the pages' mathematics fixes,
independent of how the oracle is coded:

- the chunk-wise rewrite ([LA-Infra] "Prefill中的Chunk微观并行"), coded separately in
  oracle/chunk_form.py, equals the sequential recurrence for every chunk size, including
  partial last chunks, for both gate kinds;
- the recurrence is affine in the initial state, S_T(S_0) = Transition S_0 + Delta
  ([LA-Infra] "Linear Attention Chunk-Wise"): f(a X + b Y) = a f(X) + b f(Y) + (1 - a - b) f(0);
- running a sequence in two parts, handing the state over, equals running it at once
  ([Handbook] "同一个计算的两种写法");
- a per-key gate with equal channels is the scalar gate ([LA-Infra] "KDA: By Channel的遗忘门");
- with v = 0, unit keys and gates and betas in their ranges, the state's spectral norm does
  not grow ([LA-Infra] App. 2: I - beta k k^T has eigenvalues 1 - beta and 1).
"""
import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
from oracle.chunk_form import chunked

SETTINGS = dict(max_examples=25, deadline=None,
                suppress_health_check=[HealthCheck.too_slow])


def _case(seed, lengths, H, dk, dv, perkey, unit=True):
    r = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, dv))
    a = r.standard_normal((T, H, dk) if perkey else (T, H))
    g = -np.log1p(np.exp(-(a + 2.0)))            # log sigmoid(a + 2) <= 0
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((T, H))))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return q, k, v, g, beta, cu


lengths_st = st.lists(st.integers(0, 70), min_size=1, max_size=4).filter(lambda l: sum(l) > 0)


@settings(**SETTINGS)
@given(seed=st.integers(0, 10**6), lengths=lengths_st, H=st.integers(1, 2),
       dk=st.sampled_from([2, 3, 8, 16]), dv=st.sampled_from([1, 4, 16]),
       chunk=st.sampled_from([1, 3, 16, 64]), perkey=st.booleans())
def test_chunk_form_equals_recurrence(seed, lengths, H, dk, dv, chunk, perkey):
    q, k, v, g, beta, cu = _case(seed, lengths, H, dk, dv, perkey)
    r = np.random.default_rng(seed + 1)
    init = r.standard_normal((len(lengths), H, dk, dv)) / dk ** 0.5
    o1, s1 = oracle.recurrence(q, k, v, g, beta, cu, scale=0.7, init_states=init)
    o2, s2 = chunked(q, k, v, g, beta, cu, chunk, scale=0.7, init_states=init)
    assert oracle.rel_err(o2, o1) <= 1e-10 and oracle.rel_err(s2, s1) <= 1e-10


@settings(**SETTINGS)
@given(seed=st.integers(0, 10**6), T=st.integers(1, 80), dk=st.sampled_from([2, 8, 16]),
       dv=st.sampled_from([1, 8]), perkey=st.booleans(),
       a=st.floats(-2, 2), b=st.floats(-2, 2))
def test_final_state_is_affine_in_the_initial_state(seed, T, dk, dv, perkey, a, b):
    q, k, v, g, beta, cu = _case(seed, [T], 1, dk, dv, perkey)
    r = np.random.default_rng(seed + 2)
    X, Y = r.standard_normal((2, 1, 1, dk, dv))
    f = lambda S: oracle.recurrence(q, k, v, g, beta, cu, init_states=S)
    (oX, sX), (oY, sY), (o0, s0) = f(X), f(Y), f(np.zeros_like(X))
    oZ, sZ = f(a * X + b * Y)
    assert oracle.rel_err(sZ, a * sX + b * sY + (1 - a - b) * s0) <= 1e-10
    assert oracle.rel_err(oZ, a * oX + b * oY + (1 - a - b) * o0) <= 1e-10


@settings(**SETTINGS)
@given(seed=st.integers(0, 10**6), T=st.integers(2, 100), cut=st.floats(0.0, 1.0),
       dk=st.sampled_from([4, 16]), perkey=st.booleans())
def test_split_handoff_equals_one_pass(seed, T, cut, dk, perkey):
    q, k, v, g, beta, cu = _case(seed, [T], 2, dk, dk, perkey)
    t1 = int(round(cut * T))
    o, s = oracle.recurrence(q, k, v, g, beta, cu)
    oa, sa = oracle.recurrence(q[:t1], k[:t1], v[:t1], g[:t1], beta[:t1],
                               np.array([0, t1], dtype=np.int32))
    ob, sb = oracle.recurrence(q[t1:], k[t1:], v[t1:], g[t1:], beta[t1:],
                               np.array([0, T - t1], dtype=np.int32), init_states=sa)
    assert oracle.rel_err(np.concatenate([oa, ob]), o) <= 1e-12
    assert oracle.rel_err(sb, s) <= 1e-12


@settings(**SETTINGS)
@given(seed=st.integers(0, 10**6), lengths=lengths_st, dk=st.sampled_from([2, 8, 16]),
       dv=st.sampled_from([1, 8]))
def test_equal_channel_per_key_gate_is_the_scalar_gate(seed, lengths, dk, dv):
    q, k, v, g, beta, cu = _case(seed, lengths, 2, dk, dv, False)
    gk = np.repeat(g[:, :, None], dk, axis=2)
    o1, s1 = oracle.recurrence(q, k, v, g, beta, cu)
    o2, s2 = oracle.recurrence(q, k, v, gk, beta, cu)
    assert oracle.rel_err(o2, o1) <= 1e-13 and oracle.rel_err(s2, s1) <= 1e-13


@settings(**SETTINGS)
@given(seed=st.integers(0, 10**6), T=st.integers(1, 60), dk=st.sampled_from([2, 4, 16]),
       perkey=st.booleans())
def test_zero_values_never_grow_the_state(seed, T, dk, perkey):
    q, k, v, g, beta, cu = _case(seed, [T], 1, dk, 4, perkey)
    v[:] = 0.0
    r = np.random.default_rng(seed + 3)
    S = r.standard_normal((1, 1, dk, 4))
    norm = np.linalg.norm(S[0, 0], 2)
    for t in range(T):
        _, S = oracle.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1],
                                 np.array([0, 1], dtype=np.int32), init_states=S)
        new = np.linalg.norm(S[0, 0], 2)
        assert new <= norm * (1 + 1e-12), (t, new, norm)
        norm = new
