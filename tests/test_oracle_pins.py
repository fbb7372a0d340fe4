"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it follows. None of them re-types the oracle's own loop:
they use exact rational arithmetic on the matrix form of the update, explicit matrix
products of per-token transitions, the chunk-wise form, closed forms and the pages'
printed worked examples.

Pages: [LA-Infra] "深度解析线性注意力机制演进与 AI Infra 实现"; [Handbook] "线性注意力与混合架构的推理";
[DeltaLog] "DeltaLog：延迟物化递归状态以加速线性注意力解码" reading notes.
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

import oracle
from oracle import chunk_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _random_case(seed, T, H, dk, dv, perkey=False, lengths=None, init=False):
    r = _rng(seed)
    lengths = lengths or [T]
    T = sum(lengths)
    q = _unit(r.standard_normal((T, H, dk)))
    k = _unit(r.standard_normal((T, H, dk)))
    v = r.standard_normal((T, H, dv))
    x = r.standard_normal((T, H, dk) if perkey else (T, H))
    g = -np.log1p(np.exp(-(x + 3.0)))           # log sigmoid(x + 3)
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((T, H))))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S0 = r.standard_normal((len(lengths), H, dk, dv)) / math.sqrt(dk) if init else None
    return q, k, v, g, beta, cu, S0


# ----------------------------------------------------------------- exact rational pins
def _frac_matrix_update_scalar(S, alpha, beta, k, v):
    """The gated delta rule's matrix form in d_k x d_v orientation:
    S_t = alpha (I - beta k k^T) S_{t-1} + beta k v^T."""
    dk, dv = len(S), len(S[0])
    kS = [sum(k[i] * S[i][j] for i in range(dk)) for j in range(dv)]   # k^T S
    return [[alpha * (S[i][j] - beta * k[i] * kS[j]) + beta * k[i] * v[j]
             for j in range(dv)] for i in range(dk)]


def _frac_matrix_update_perkey(S, alpha, beta, k, v):
    """Per-key form: S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T
    ([LA-Infra] "KDA: By Channel的遗忘门", transposed to d_k x d_v)."""
    dk, dv = len(S), len(S[0])
    DS = [[alpha[i] * S[i][j] for j in range(dv)] for i in range(dk)]
    kDS = [sum(k[i] * DS[i][j] for i in range(dk)) for j in range(dv)]
    return [[DS[i][j] - beta * k[i] * kDS[j] + beta * k[i] * v[j]
             for j in range(dv)] for i in range(dk)]


RAT_KEYS = [(Fr(3, 5), Fr(4, 5), Fr(0)), (Fr(0), Fr(3, 5), Fr(4, 5)),
            (Fr(4, 5), Fr(0), Fr(3, 5)), (Fr(1, 3), Fr(2, 3), Fr(2, 3)),
            (Fr(2, 7), Fr(3, 7), Fr(6, 7)), (Fr(1, 2), Fr(-1, 3), Fr(1, 4))]  # last: not unit
RAT_Q = [(Fr(1), Fr(-2), Fr(1, 2)), (Fr(2, 3), Fr(0), Fr(1)), (Fr(-1, 4), Fr(1), Fr(3, 2)),
         (Fr(1, 5), Fr(1, 5), Fr(-1)), (Fr(1), Fr(1), Fr(1)), (Fr(0), Fr(-1, 2), Fr(2))]
RAT_V = [(Fr(1), Fr(-1)), (Fr(2), Fr(1, 2)), (Fr(-3, 2), Fr(1)), (Fr(1, 4), Fr(2)),
         (Fr(-1), Fr(-1, 3)), (Fr(5, 4), Fr(0))]
RAT_ALPHA = [Fr(1, 2), Fr(3, 4), Fr(1), Fr(7, 8), Fr(2, 3), Fr(9, 10)]
RAT_BETA = [Fr(1), Fr(1, 2), Fr(3, 4), Fr(0), Fr(1, 3), Fr(2, 5)]


@pytest.mark.parametrize("scale", [Fr(1), Fr(1, 2)])
def test_rational_exact_scalar_gate(scale):
    """[LA-Infra] "GDN：增加遗忘门" matrix form, exact rationals vs fp64 oracle."""
    T, dk, dv = 6, 3, 2
    S = [[Fr(i - j, 3) for j in range(dv)] for i in range(dk)]          # nonzero S0
    S0 = np.array([[float(x) for x in row] for row in S])
    outs = []
    for t in range(T):
        S = _frac_matrix_update_scalar(S, RAT_ALPHA[t], RAT_BETA[t], RAT_KEYS[t], RAT_V[t])
        outs.append([scale * sum(S[i][j] * RAT_Q[t][i] for i in range(dk)) for j in range(dv)])
    f = lambda a: np.array(a, dtype=np.float64)
    q = f([[float(x) for x in r] for r in RAT_Q])[:, None, :]
    k = f([[float(x) for x in r] for r in RAT_KEYS])[:, None, :]
    v = f([[float(x) for x in r] for r in RAT_V])[:, None, :]
    g = np.log(f([float(a) for a in RAT_ALPHA]))[:, None]
    beta = f([float(b) for b in RAT_BETA])[:, None]
    o, st = oracle.recurrence(q, k, v, g, beta, [0, T], scale=float(scale),
                              init_states=S0[None, None])
    exp_o = f([[float(x) for x in r] for r in outs])
    exp_s = f([[float(x) for x in r] for r in S])
    assert np.max(np.abs(o[:, 0] - exp_o)) < 1e-14
    assert np.max(np.abs(st[0, 0] - exp_s)) < 1e-14


def test_rational_exact_per_key_gate():
    """[LA-Infra] "KDA: By Channel的遗忘门": per-key decay acts on key rows, correction against
    the decayed state; exact rationals vs fp64 oracle."""
    T, dk, dv = 6, 3, 2
    alphas = [(Fr(1, 2), Fr(3, 4), Fr(1)), (Fr(1), Fr(1, 4), Fr(2, 3)),
              (Fr(5, 6), Fr(5, 6), Fr(1, 2)), (Fr(9, 10), Fr(1), Fr(3, 5)),
              (Fr(1, 3), Fr(2, 3), Fr(1)), (Fr(7, 8), Fr(1, 8), Fr(1, 2))]
    S = [[Fr(2 * i + j + 1, 5) for j in range(dv)] for i in range(dk)]
    S0 = np.array([[float(x) for x in row] for row in S])
    outs = []
    for t in range(T):
        S = _frac_matrix_update_perkey(S, alphas[t], RAT_BETA[t], RAT_KEYS[t], RAT_V[t])
        outs.append([sum(S[i][j] * RAT_Q[t][i] for i in range(dk)) for j in range(dv)])
    f = lambda a: np.array(a, dtype=np.float64)
    q = f([[float(x) for x in r] for r in RAT_Q])[:, None, :]
    k = f([[float(x) for x in r] for r in RAT_KEYS])[:, None, :]
    v = f([[float(x) for x in r] for r in RAT_V])[:, None, :]
    g = np.log(f([[float(a) for a in r] for r in alphas]))[:, None, :]
    beta = f([float(b) for b in RAT_BETA])[:, None]
    o, st = oracle.recurrence(q, k, v, g, beta, [0, T], init_states=S0[None, None])
    assert np.max(np.abs(o[:, 0] - f([[float(x) for x in r] for r in outs]))) < 1e-14
    assert np.max(np.abs(st[0, 0] - f([[float(x) for x in r] for r in S]))) < 1e-14


# ------------------------------------------------------ affine product form (brute force)
@pytest.mark.parametrize("perkey", [False, True])
def test_affine_transition_product(perkey):
    """[LA-Infra] "Linear Attention Chunk-Wise": each token is an affine map
    S_t = T_t S_{t-1} + H_t (here T_t = (I - beta k k^T) Diag(alpha_t), H_t = beta k v^T); the
    whole sequence is Transition S_0 + Delta with Transition the ordered product of T_t."""
    T, dk, dv = 40, 6, 5
    q, k, v, g, beta, cu, S0 = _random_case(1, T, 1, dk, dv, perkey=perkey, init=True)
    Tr = np.eye(dk)
    Dl = np.zeros((dk, dv))
    outs = []
    for t in range(T):
        a = np.exp(g[t, 0]) * np.ones(dk)
        Tt = (np.eye(dk) - beta[t, 0] * np.outer(k[t, 0], k[t, 0])) @ np.diag(a)
        Ht = beta[t, 0] * np.outer(k[t, 0], v[t, 0])
        Tr = Tt @ Tr
        Dl = Tt @ Dl + Ht
        outs.append((Tr @ S0[0, 0] + Dl).T @ q[t, 0])
    o, st = oracle.recurrence(q, k, v, g, beta, cu, init_states=S0)
    assert np.max(np.abs(o[:, 0] - np.array(outs))) < 1e-12
    assert np.max(np.abs(st[0, 0] - (Tr @ S0[0, 0] + Dl))) < 1e-12


# ------------------------------------------------------------ segment composition
@pytest.mark.parametrize("perkey", [False, True])
@pytest.mark.parametrize("bounds", [[0, 23, 50], [0, 9, 20, 31, 50], [0, 7, 13, 20, 27, 33, 40, 46, 50]])
def test_segment_composition(perkey, bounds):
    """[LA-Infra] "Linear Attention Chunk-Wise": every output and the final state are affine in
    the incoming state, so a sequence cut into segments is rebuilt from per-segment runs of
    the recurrence alone: a run from a zero state with the real v (outputs O0_j, final state
    Delta_j) and a run from the identity with v = 0 (outputs L_j, final state, the
    transition, P_j), then S_(j+1) = P_j S_j + Delta_j and O = O0_j + L_j S_j. This is the
    composition the segmented scan evaluates; 2, 4 and 8 segments against one pass."""
    T, dk, dv = bounds[-1], 6, 5
    q, k, v, g, beta, cu, S0 = _random_case(9, T, 1, dk, dv, perkey=perkey, init=True)
    o_ref, s_ref = oracle.recurrence(q, k, v, g, beta, cu, scale=0.7, init_states=S0)
    S = S0[0, 0]
    o = np.zeros_like(o_ref)
    for a, b in zip(bounds[:-1], bounds[1:]):
        part = np.array([0, b - a], dtype=np.int32)
        o0, dl = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], part, scale=0.7)
        lo, p = oracle.recurrence(q[a:b], k[a:b], np.zeros((b - a, 1, dk)), g[a:b], beta[a:b],
                                  part, scale=0.7, init_states=np.eye(dk)[None, None])
        o[a:b, 0] = o0[:, 0] + lo[:, 0] @ S
        S = p[0, 0] @ S + dl[0, 0]
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(S - s_ref[0, 0])) < 1e-12


# ------------------------------------------------------------------- chunk-wise form
@pytest.mark.parametrize("perkey", [False, True])
@pytest.mark.parametrize("chunk", [16, 32, 64, 5])
def test_chunk_form_matches_recurrence(perkey, chunk):
    """[LA-Infra] "Prefill中的Chunk微观并行" (six-step order) is an exact rewrite of the
    recurrence; chunks restart at sequence boundaries; last chunks may be short."""
    lengths = [70, 1, 33, 64]
    q, k, v, g, beta, cu, S0 = _random_case(2, 0, 2, 16, 8, perkey=perkey,
                                            lengths=lengths, init=True)
    o_ref, s_ref = oracle.recurrence(q, k, v, g, beta, cu, scale=0.3, init_states=S0)
    o_ch, s_ch = chunk_form.chunked(q, k, v, g, beta, cu, chunk, scale=0.3, init_states=S0)
    assert oracle.rel_err(o_ch, o_ref) < 1e-12
    assert oracle.rel_err(s_ch, s_ref) < 1e-12


def test_first_token_identity():
    """[LA-Infra] "块内输出" check at i = 1: o_1 = S_0^T (q_1 * alpha_1) + (q_1 . k_1) r_1."""
    q, k, v, g, beta, cu, S0 = _random_case(3, 1, 1, 8, 4, perkey=True, init=True)
    a = np.exp(g[0, 0])
    S0m = S0[0, 0]
    r1 = beta[0, 0] * (v[0, 0] - (a[:, None] * S0m).T @ k[0, 0])
    expect = S0m.T @ (q[0, 0] * a) + np.dot(q[0, 0], k[0, 0]) * r1
    o, _ = oracle.recurrence(q, k, v, g, beta, cu, init_states=S0)
    assert np.max(np.abs(o[0, 0] - expect)) < 1e-14


# ------------------------------------------------------------------- special cases
def _gla_recurrent(q, k, v, alpha):
    """[Handbook] "同一个计算的两种写法": S_t = alpha_t S_{t-1} + k_t^T v_t, o_t = q_t S_t."""
    S = np.zeros((q.shape[1], v.shape[1]))
    out = []
    for t in range(q.shape[0]):
        S = alpha[t] * S + np.outer(k[t], v[t])
        out.append(q[t] @ S)
    return np.array(out), S


def _gla_chunked(q, k, v, alpha, C):
    """The same GLA map evaluated chunk by chunk: inside a chunk a causal C x C product
    with the decay between positions, across chunks only the state is carried."""
    T = q.shape[0]
    S = np.zeros((q.shape[1], v.shape[1]))
    out = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(T, s + C)
        lg = np.cumsum(np.log(alpha[s:e]))
        dec = np.tril(np.exp(lg[:, None] - np.where(
            np.tril(np.ones((e - s, e - s))) > 0, lg[None, :], np.inf)))
        out[s:e] = (q[s:e] @ k[s:e].T * dec) @ v[s:e] + np.exp(lg)[:, None] * (q[s:e] @ S)
        S = np.exp(lg[-1]) * S + (np.exp(lg[-1] - lg)[:, None] * k[s:e]).T @ v[s:e]
    return out, S


def test_handbook_gla_toy_recurrent_equals_chunked():
    """[Handbook] "同一个计算的两种写法": seed 0, T=64, d=16, C=16; the page prints that the
    recurrent and chunked GLA outputs and final states agree at atol 1e-5 ("True / True")."""
    torch.manual_seed(0)
    T, D, C = 64, 16, 16
    q, k, v = torch.randn(T, D) / 4, torch.randn(T, D) / 4, torch.randn(T, D)
    alpha = torch.sigmoid(torch.randn(T) + 3)
    q, k, v, alpha = (x.double().numpy() for x in (q, k, v, alpha))
    o1, s1 = _gla_recurrent(q, k, v, alpha)
    o2, s2 = _gla_chunked(q, k, v, alpha, C)
    assert np.allclose(o1, o2, atol=1e-5) and np.allclose(s1, s2, atol=1e-5)


def test_gdn_reduces_to_gla_with_orthogonal_keys():
    """With mutually orthogonal keys, zero initial state and beta = 1 the delta correction
    reads nothing (A = 0, R = I in [LA-Infra] "计算 Δchunk"), so GDN equals the handbook's GLA
    recurrence with the same alpha."""
    torch.manual_seed(0)
    T = D = 16
    q, k, v = torch.randn(T, D) / 4, torch.randn(T, D) / 4, torch.randn(T, D)
    alpha = torch.sigmoid(torch.randn(T) + 3)
    q, k, v, alpha = (x.double().numpy() for x in (q, k, v, alpha))
    Qm, _ = np.linalg.qr(k.T)                  # orthonormal columns
    k = Qm.T.copy()
    o_gla, s_gla = _gla_recurrent(q, k, v, alpha)
    o_ch, s_ch = _gla_chunked(q, k, v, alpha, 4)
    o, st = oracle.recurrence(q[:, None], k[:, None], v[:, None], np.log(alpha)[:, None],
                              np.ones((T, 1)), [0, T])
    assert np.max(np.abs(o[:, 0] - o_gla)) < 1e-13
    assert np.max(np.abs(st[0, 0] - s_gla)) < 1e-13
    assert np.max(np.abs(o_ch - o_gla)) < 1e-12


def test_beta_zero_closed_form():
    """beta = 0 writes nothing: S_t = (prod alpha) S_0 and o_t = s (prod_{tau<=t} alpha) S_0^T q_t."""
    q, k, v, g, beta, cu, S0 = _random_case(4, 30, 2, 8, 6, init=True)
    beta[:] = 0.0
    o, st = oracle.recurrence(q, k, v, g, beta, cu, scale=0.7, init_states=S0)
    cum = np.exp(np.cumsum(g, axis=0))                                  # [T, H]
    expect = 0.7 * cum[:, :, None] * np.einsum("hkv,thk->thv", S0[0], q)
    assert np.max(np.abs(o - expect)) < 1e-13
    assert np.max(np.abs(st[0] - cum[-1][:, None, None] * S0[0])) < 1e-13


def test_delta_rule_overwrite_and_interpolation():
    """[LA-Infra] "从训练的角度理解演进" / App. 2: with ||k|| = 1 the read along the written key
    becomes (1 - beta) Sbar^T k + beta v; beta = 1 overwrites exactly."""
    q, k, v, g, beta, cu, S0 = _random_case(5, 12, 1, 8, 5, init=True)
    o_prev, s_prev = oracle.recurrence(q[:-1], k[:-1], v[:-1], g[:-1], beta[:-1],
                                       [0, 11], init_states=S0)
    for b in (1.0, 0.35):
        bb = beta.copy()
        bb[-1] = b
        qq = q.copy()
        qq[-1] = k[-1]                                  # read along the written key
        o, _ = oracle.recurrence(qq, k, v, g, bb, cu, init_states=S0)
        sbar_k = np.exp(g[-1, 0]) * s_prev[0, 0].T @ k[-1, 0]
        expect = (1 - b) * sbar_k + b * v[-1, 0]
        assert np.max(np.abs(o[-1, 0] - expect)) < 1e-13


def test_orthogonal_query_unaffected_by_write():
    """[LA-Infra] App. 2 "查询完全无关的知识": a query orthogonal to k_t reads Sbar_t^T q."""
    q, k, v, g, beta, cu, S0 = _random_case(6, 9, 1, 8, 4, perkey=True, init=True)
    _, s_prev = oracle.recurrence(q[:-1], k[:-1], v[:-1], g[:-1], beta[:-1], [0, 8],
                                  init_states=S0)
    kk = k[-1, 0]
    qo = np.random.default_rng(0).standard_normal(8)
    qo -= np.dot(qo, kk) / np.dot(kk, kk) * kk
    qq = q.copy()
    qq[-1, 0] = qo
    o, _ = oracle.recurrence(qq, k, v, g, beta, cu, init_states=S0)
    sbar = np.exp(g[-1, 0])[:, None] * s_prev[0, 0]
    assert np.max(np.abs(o[-1, 0] - sbar.T @ qo)) < 1e-13


@pytest.mark.parametrize("perkey", [False, True])
def test_non_expansion(perkey):
    """[LA-Infra] App. 2: with unit keys, 0 <= beta <= 1 and 0 <= alpha <= 1 the transition
    does not enlarge the state: with v = 0 the spectral norm never grows."""
    r = _rng(7)
    T, dk, dv = 25, 6, 6
    q, k, v, g, beta, cu, S0 = _random_case(7, T, 1, dk, dv, perkey=perkey, init=True)
    v[:] = 0.0
    beta[:] = r.uniform(0, 1, beta.shape)
    prev = np.linalg.norm(S0[0, 0], 2)
    S = S0
    for t in range(T):
        _, S = oracle.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                 beta[t:t + 1], [0, 1], init_states=S)
        cur = np.linalg.norm(S[0, 0], 2)
        assert cur <= prev * (1 + 1e-12)
        prev = cur


def test_split_prefill_handoff_and_decode():
    """[Handbook] "在真实模型上核对": splitting a prompt and handing the state over (also
    token-by-token, i.e. decode steps) gives the one-shot result."""
    q, k, v, g, beta, cu, S0 = _random_case(8, 64, 2, 8, 8, init=True)
    o_all, s_all = oracle.recurrence(q, k, v, g, beta, cu, init_states=S0)
    S = S0
    parts = []
    for a, b in ((0, 20), (20, 45), (45, 64)):
        o, S = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a],
                                 init_states=S)
        parts.append(o)
    assert np.array_equal(np.concatenate(parts), o_all) and np.array_equal(S, s_all)
    S = S0
    for t in range(64):
        o, S = oracle.decode_step(q[t][None], k[t][None], v[t][None], g[t][None],
                                  beta[t][None], S)
        assert np.array_equal(o[0], o_all[t])


def test_per_key_equal_channels_is_scalar_gate():
    """[LA-Infra] "KDA: By Channel的遗忘门": a per-key gate with all channels equal is GDN's
    scalar gate."""
    q, k, v, g, beta, cu, S0 = _random_case(9, 40, 2, 8, 4, init=True)
    gk = np.repeat(g[:, :, None], 8, axis=2)
    o1, s1 = oracle.recurrence(q, k, v, g, beta, cu, init_states=S0)
    o2, s2 = oracle.recurrence(q, k, v, gk, beta, cu, init_states=S0)
    assert np.max(np.abs(o1 - o2)) < 1e-15 and np.max(np.abs(s1 - s2)) < 1e-15


def test_in_kernel_l2norm_reading():
    """[LA-Infra] App. 2 "L2 Norm是什么": x / sqrt(x.x + eps) (eps guard, value unstated on the
    page; 1e-6 here). Normalising inside equals feeding normalised inputs."""
    r = _rng(10)
    T, H, d = 17, 2, 8
    q = r.standard_normal((T, H, d)) * 3
    k = r.standard_normal((T, H, d)) * 0.2
    v = r.standard_normal((T, H, d))
    g = -r.uniform(0, 0.5, (T, H))
    beta = r.uniform(0, 1, (T, H))
    nq = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    nk = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    o1, s1 = oracle.recurrence(q, k, v, g, beta, [0, T], l2norm=True, eps=1e-6)
    o2, s2 = oracle.recurrence(nq, nk, v, g, beta, [0, T])
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(s1 - s2)) < 1e-13


# ------------------------------------------------------------- appendix 1 numerics
def test_appendix1_naive_split_overflows_reference_split_does_not():
    """[LA-Infra] "附1. chunk内 A和M 的计算": with a per-key log gate of -5 per step the
    in-chunk cumulative gate reaches 64 * (-5) = -320, exp(320) exceeds fp32 (about e^88.7)
    and the split exp(G_i) exp(-G_j) overflows; the 16 x 16 reference-point split stays finite
    and matches the fp64 definition."""
    r = _rng(11)
    C, dk = 64, 128
    K = _unit(r.standard_normal((C, dk)))
    Q = _unit(r.standard_normal((C, dk)))
    g = np.full((C, dk), -5.0)
    beta = r.uniform(0, 1, C)
    A_n, M_n = chunk_form.a_and_m_naive_split(K, Q, g, beta)
    assert not np.all(np.isfinite(A_n)) or not np.all(np.isfinite(M_n))
    A_r, M_r = chunk_form.a_and_m_reference_split(K, Q, g, beta)
    assert np.all(np.isfinite(A_r)) and np.all(np.isfinite(M_r))
    _, _, inter = chunk_form.chunk_step(np.zeros((dk, 4)), K, Q, np.zeros((C, 4)), g, beta, 1.0)
    assert np.max(np.abs(A_r - inter["A"])) < 1e-6 * max(1.0, np.max(np.abs(inter["A"])))
    assert np.max(np.abs(M_r - inter["M"])) < 1e-6 * max(1.0, np.max(np.abs(inter["M"])))
    # the diagonal-block positive exponent stays below e^75 for 15 steps of -5
    assert 15 * 5 < 88


def test_reference_split_matches_definition_random_gates():
    r = _rng(12)
    C, dk = 48, 32
    K, Q = r.standard_normal((C, dk)), r.standard_normal((C, dk))
    g = -r.uniform(0, 3, (C, dk))
    beta = r.uniform(0, 1, C)
    A_r, M_r = chunk_form.a_and_m_reference_split(K, Q, g, beta, dtype=np.float64)
    _, _, inter = chunk_form.chunk_step(np.zeros((dk, 2)), K, Q, np.zeros((C, 2)), g, beta, 1.0)
    assert np.max(np.abs(A_r - inter["A"])) < 1e-12
    assert np.max(np.abs(M_r - inter["M"])) < 1e-12


# ----------------------------------------------------------------------- DeltaLog
def test_deltalog_scalar_worked_example():
    """[DeltaLog] §2.3 teaching example (golden): scalar state, S0 = 10, decay 1/2,
    increments 2, 3, 4, M = 3 -> logical 7, 6.5, 7.25; base 10, 10, 7.25."""
    ex = json.load(open(os.path.join(GOLDEN, "deltalog_scalar_example.json")))
    st = oracle.DeltaLogState(np.array([[[ex["S0"]]]]), M=ex["M"])
    for t, inc in enumerate(ex["increments"]):
        o = st.step(np.ones((1, 1)), np.ones((1, 1)), np.array([[inc]]),
                    np.array([[math.log(ex["decay"])]]), np.ones(1), mode=1, klog_bf16=False)
        assert abs(o[0, 0] - ex["logical_state"][t]) < 1e-13
        assert abs(st.base[0, 0, 0] - ex["base"][t]) < 1e-13
        assert abs(st.materialize()[0, 0, 0] - ex["logical_state"][t]) < 1e-13


@pytest.mark.parametrize("perkey", [False, True])
@pytest.mark.parametrize("M", [2, 3, 8])
def test_deltalog_invariant_equals_dense(perkey, M):
    """[DeltaLog] §2.2 Eq. (7) and §2.3 Algorithm 1: after every step (append or merge) the
    materialised base + log equals the dense recurrent state, and the outputs agree."""
    n, dk, dv, T = 5, 8, 6, 20
    r = _rng(13)
    base0 = r.standard_normal((n, dk, dv)) / math.sqrt(dk)
    st = oracle.DeltaLogState(base0, M=M, perkey=perkey)
    S = base0[:, None].copy()
    for t in range(T):
        q = _unit(r.standard_normal((n, dk)))
        k = _unit(r.standard_normal((n, dk)))
        v = r.standard_normal((n, dv))
        g = -r.uniform(0.0, 0.3, (n, dk) if perkey else (n,))
        beta = r.uniform(0, 1, n)
        o_dl = st.step(q, k, v, g, beta, scale=0.5, klog_bf16=False)
        o_d, S2 = oracle.decode_step(q[:, None], k[:, None], v[:, None], g[:, None],
                                     beta[:, None], S.reshape(n, 1, dk, dv), scale=0.5)
        S = S2.reshape(n, 1, dk, dv)
        assert np.max(np.abs(o_dl - o_d[:, 0])) < 1e-13
        assert np.max(np.abs(st.materialize() - S[:, 0])) < 1e-13
        assert np.all(st.len == (t + 1) % M)


def test_deltalog_bf16_keys_exact_for_bf16_inputs():
    """[DeltaLog] §2.7: K_log is bf16. Keys that are already bf16 values are logged exactly,
    so base + log still equals the dense state; fp32 keys are rounded (small deviation)."""
    n, dk, dv = 3, 16, 4
    r = _rng(14)
    base0 = r.standard_normal((n, dk, dv))
    st = oracle.DeltaLogState(base0, M=4)
    S = base0[:, None].copy()
    for t in range(6):
        k = torch.tensor(_unit(r.standard_normal((n, dk)))).to(torch.bfloat16).double().numpy()
        q = _unit(r.standard_normal((n, dk)))
        v = r.standard_normal((n, dv))
        g = -r.uniform(0, 0.2, n)
        beta = r.uniform(0, 1, n)
        o_dl = st.step(q, k, v, g, beta, klog_bf16=True)
        o_d, S2 = oracle.decode_step(q[:, None], k[:, None], v[:, None], g[:, None],
                                     beta[:, None], S.reshape(n, 1, dk, dv))
        S = S2.reshape(n, 1, dk, dv)
        assert np.max(np.abs(o_dl - o_d[:, 0])) < 1e-12
    assert np.max(np.abs(st.klog[:, :2] - torch.tensor(st.klog[:, :2]).float()
                         .to(torch.bfloat16).double().numpy())) == 0.0


def test_deltalog_fp32_keys_logged_as_bf16():
    """[DeltaLog] §2.7: K_log is bf16. fp32 keys are logged as their round-to-nearest-even
    bf16 values (torch's conversion as the independent rounding), not as the raw keys."""
    n, dk, dv, M = 4, 32, 4, 5
    r = _rng(15)
    st = oracle.DeltaLogState(r.standard_normal((n, dk, dv)), M=M)
    ks = []
    for t in range(M - 1):
        k = torch.tensor(_unit(r.standard_normal((n, dk)))).float().double().numpy()
        ks.append(k)
        st.step(_unit(r.standard_normal((n, dk))), k, r.standard_normal((n, dv)),
                -r.uniform(0, 0.2, n), r.uniform(0, 1, n), klog_bf16=True)
    ks = np.stack(ks, 1)
    want = torch.tensor(ks).float().to(torch.bfloat16).double().numpy()
    assert np.any(want != ks)
    assert np.array_equal(st.klog, want)


def test_deltalog_capacity_table():
    """[DeltaLog] §2.5 capacity table (golden): 21.125 / 17 / 14 MiB at B = 128."""
    from gated_delta_rule_prefill_amd.traffic import DeltaLogModel
    tab = json.load(open(os.path.join(GOLDEN, "deltalog_capacity.json")))
    for row in tab["rows"]:
        m = DeltaLogModel(tab["B"], tab["H"], tab["dk"], tab["dv"], row["M"],
                          d_lambda=row["d_lambda"], p_K=row["p_K"], p_U=row["p_U"])
        assert m.aux_bytes() / 2 ** 20 == pytest.approx(row["aux_MiB"], abs=1e-9)
        assert 100 * m.aux_bytes() / m.c_state == pytest.approx(row["vs_base_pct"], abs=0.006)


def test_deltalog_traffic_bound():
    """[DeltaLog] §2.5: ignoring log and common traffic, dense / DeltaLog = 2 / (1 + 1/M),
    about 1.78x at M = 8; and the full model says the M = 8 GDN log is profitable."""
    from gated_delta_rule_prefill_amd.traffic import DeltaLogModel
    gold = json.load(open(os.path.join(GOLDEN, "deltalog_traffic.json")))
    m = DeltaLogModel(gold["B"], gold["H"], gold["dk"], gold["dv"], gold["M"])
    bound = (2 * m.c_state) / (m.c_state + m.c_state / m.M)
    assert bound == pytest.approx(gold["state_only_bound"], abs=0.005)
    assert m.profitable() and m.t_dense() / m.t_delta() < bound


# ------------------------------------------------------------------------ conv1d
def test_conv1d_silu_against_numpy_convolve():
    """[LA-Infra] "去掉分母引入卷积": per-channel causal window of 4 (weight column 3 on the
    current token, column 0 on the token three back) then SiLU; zero history per sequence.
    Checked against numpy.convolve per channel and sequence."""
    r = _rng(15)
    lengths = [5, 1, 9, 3]
    T, ch, W = sum(lengths), 7, 4
    x = r.standard_normal((T, ch))
    w = r.standard_normal((ch, W))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    y = oracle.conv1d_silu(x, w, cu)
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        for c in range(ch):
            full = np.convolve(x[a:b, c], w[c, ::-1])[: b - a]
            assert np.max(np.abs(y[a:b, c] - full / (1 + np.exp(-full)))) < 1e-13
    # the page's literal 4-term formula at one interior position
    t, c = cu[2] + 5, 3
    z = sum(x[t - 3 + j, c] * w[c, j] for j in range(4))
    assert abs(y[t, c] - z / (1 + math.exp(-z))) < 1e-13


# ------------------------------------------------------------------------ KDA gate formula
def test_kda_gate_hand_values_and_broadcast():
    """[LA-Infra] KDA实现逻辑概述: forget_log = lower_bound * sigmoid(e^{A_log} (forget_b +
    dt_bias)), A_log per head, dt_bias per (head, channel). H = 2, d_k = 2 with A_log =
    [0, ln 2], dt_bias = [[0, 1], [2, 3]], forget_b = 0 gives z = [[0, 1], [4, 6]]; the values
    are -5 sigmoid(z) evaluated by hand."""
    from oracle.gates import kda_forget_log
    got = kda_forget_log(np.zeros((2, 2)), [[0.0, 1.0], [2.0, 3.0]], [0.0, np.log(2.0)], -5.0)
    want = [[-2.5, -3.6552928931500244], [-4.910068950189542, -4.987636884216827]]
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # a leading batch axis broadcasts; forget_b shifts x per channel
    fb = np.array([[[1.0, 0.0], [0.0, 0.0]]])
    got = kda_forget_log(fb, np.zeros((2, 2)), [0.0, 0.0], -5.0)
    assert got.shape == (1, 2, 2)
    assert np.allclose(got[0, 0], [-3.6552928931500244, -2.5], rtol=0, atol=1e-15)


def test_kda_gate_range_and_page_bound():
    """forget_log stays in (lower_bound, 0) and z = 0 gives lower_bound / 2; with
    lower_bound = -5 the decay cannot drop below e^{-5}, the ~0.67 % per step the page quotes."""
    from oracle.gates import kda_forget_log, sigmoid
    rng = np.random.default_rng(0)
    fb = rng.normal(0, 1, (64, 4, 16))
    fl = kda_forget_log(fb, rng.normal(0, 1, (4, 16)), rng.normal(0, 0.5, 4), -5.0)
    assert np.all(fl < 0) and np.all(fl > -5.0)
    # far out the sigmoid rounds to 0 or 1 in fp64: the interval closes, never overshoots
    fl = kda_forget_log(rng.normal(0, 40, (64, 4, 16)), np.zeros((4, 16)), np.ones(4), -5.0)
    assert np.all(fl <= 0) and np.all(fl >= -5.0)
    assert kda_forget_log(np.array([[0.7]]), [[-0.7]], [1.3], -3.0)[0, 0] == -1.5
    big = kda_forget_log(np.array([[60.0]]), [[0.0]], [0.0], -5.0)[0, 0]
    assert abs(np.exp(big) - np.exp(-5.0)) < 1e-15
    assert round(100 * np.exp(-5.0), 2) == 0.67
    # monotone: a larger gate projection decays more
    assert kda_forget_log(np.array([[1.0]]), [[0.0]], [0.0], -5.0)[0, 0] < \
        kda_forget_log(np.array([[0.5]]), [[0.0]], [0.0], -5.0)[0, 0]
    # write gate beta = sigmoid(logit): sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4
    assert sigmoid(0.0) == 0.5 and abs(sigmoid(np.log(3.0)) - 0.75) < 1e-15

