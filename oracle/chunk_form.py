"""Chunk-wise form of the gated delta rule in plain fp64 numpy (test infrastructure only).

This is the second of the two equivalent forms the pages derive; the tests use it to pin the
sequential recurrence in ``gdn_oracle.c`` (two independent codings of what the pages state
must agree to rounding), and to inspect intermediates. The product path never imports it.

Source: [LA-Infra] = "深度解析线性注意力机制演进与 AI Infra 实现" (todayforai.com),
section "Prefill中的Chunk微观并行", sub-sections "计算 Δchunk", "计算 Transitionchunk",
"块内输出", "完整计算顺序" (six-step order), and appendix "附1. chunk内 A和M 的计算".
The page writes the state as d_v x d_k; here it is d_k x d_v (S^T of the page), so the
page's S_0 Diag(.) becomes Diag(.) S_0 and the page's E^T K_g becomes K_g^T E.

Every quantity follows the page's names: G (in-chunk cumulative log gate), K_in, K_g,
D_C, A, R = (I + A)^{-1}, U, W, E, Q_in (the page's Q-hat_in), M, O.
"""
import numpy as np


def _exp_pair(G, i, j):
    """exp(G_i - G_j): the decay accumulated by steps j+1..i (scalar or per-channel)."""
    return np.exp(G[i] - G[j])


def chunk_step(S0, K, Q, V, g, beta, scale):
    """One chunk, one head. S0 [dk, dv]; K, Q [C, dk]; V [C, dv]; g [C] or [C, dk];
    beta [C]. Returns (O [C, dv], S_C [dk, dv], intermediates dict)."""
    S0, K, Q, V, g, beta = (np.asarray(x, dtype=np.float64) for x in (S0, K, Q, V, g, beta))
    C, dk = K.shape
    perkey = g.ndim == 2
    # Step 1: cumulative log-gate along tokens, restarting at the chunk start.
    G = np.cumsum(g, axis=0)
    Gc = G[-1]
    Gcol = G if perkey else G[:, None]          # broadcast a scalar gate over key channels
    # Step 2: two gated copies of the keys and the whole-chunk decay.
    K_in = K * np.exp(Gcol)                      # decay from the chunk start through token i
    K_g = K * np.exp(Gc - Gcol)                  # decay after token i to the chunk end
    D_C = np.exp(Gc) * np.ones(dk)               # per key channel (constant for a scalar gate)
    # Step 3: A (strictly lower) from the decayed key-key alignment, times beta_i.
    A = np.zeros((C, C))
    for i in range(C):
        for j in range(i):
            A[i, j] = beta[i] * np.dot(K[j] * _exp_pair(Gcol, i, j), K[i])
    R = np.linalg.inv(np.eye(C) + A)
    # Step 4: local residuals and the correction directions, one R for both.
    U = R @ (beta[:, None] * V)
    W = R @ (beta[:, None] * K_in)
    # Step 5: real residuals with the incoming state, then the chunk-end state.
    E = U - W @ S0
    S_C = D_C[:, None] * S0 + K_g.T @ E
    # Step 6: outputs from the decayed incoming state plus in-chunk writes (diagonal kept).
    Qh = scale * Q
    Q_in = Qh * np.exp(Gcol)
    M = np.zeros((C, C))
    for i in range(C):
        for j in range(i + 1):
            M[i, j] = np.dot(Qh[i] * _exp_pair(Gcol, i, j), K[j])
    O = Q_in @ S0 + M @ E
    inter = dict(G=G, K_in=K_in, K_g=K_g, D_C=D_C, A=A, R=R, U=U, W=W, E=E, Q_in=Q_in, M=M)
    return O, S_C, inter


def chunked(q, k, v, g, beta, cu_seqlens, chunk, scale=1.0, init_states=None):
    """Chunk-wise evaluation over packed varlen sequences (chunks restart at each sequence
    boundary; a sequence's last chunk may be short). Shapes as oracle.recurrence."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    cu = np.asarray(cu_seqlens)
    T, H, dk = q.shape
    dv = v.shape[2]
    n = len(cu) - 1
    states = (np.zeros((n, H, dk, dv)) if init_states is None
              else np.array(init_states, dtype=np.float64))
    o = np.zeros((T, H, dv))
    for s in range(n):
        for h in range(H):
            S = states[s, h]
            for c0 in range(int(cu[s]), int(cu[s + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[s + 1]))
                O, S, _ = chunk_step(S, k[c0:c1, h], q[c0:c1, h], v[c0:c1, h], g[c0:c1, h],
                                     beta[c0:c1, h], scale)
                o[c0:c1, h] = O
            states[s, h] = S
    return o, states


def a_and_m_naive_split(K, Q, g, beta, dtype=np.float32):
    """A and M from one matrix product after splitting exp(G_i - G_j) = exp(G_i) exp(-G_j)
    per channel, in `dtype` ([LA-Infra] appendix 1, part 1: exact in exact arithmetic, but
    exp(-G_j) overflows once the in-chunk cumulative gate falls below about -88)."""
    K, Q, g, beta = (np.asarray(x, dtype=dtype) for x in (K, Q, g, beta))
    G = np.cumsum(g, axis=0, dtype=dtype)
    with np.errstate(over="ignore", invalid="ignore"):
        left_k = K * np.exp(G)
        left_q = Q * np.exp(G)
        right = K * np.exp(-G)
        AK = left_k @ right.T
        MQ = left_q @ right.T
    C = K.shape[0]
    A = np.tril(AK, -1) * beta[:, None]
    M = np.tril(MQ)
    return A.astype(dtype), M.astype(dtype)


def a_and_m_reference_split(K, Q, g, beta, block=16, dtype=np.float32):
    """A and M in block x block sub-blocks ([LA-Infra] appendix 1, parts 2-3).
    Off-diagonal sub-block (a > b): reference point n = first token of row block a,
      (K_a * e^{G_a - G_n}) (K_b * e^{G_n - G_b})^T, both exponents <= 0.
    Diagonal sub-block: computed column by column, exactly, from exp(G_i - G_j) with the
      mask applied before the exponential (no positive exponent is ever formed).
    The key-side factor K_b * e^{G_n - G_b} is shared by A (row side K) and M (row side Q)."""
    K, Q, g, beta = (np.asarray(x, dtype=dtype) for x in (K, Q, g, beta))
    C, dk = K.shape
    G = np.cumsum(g, axis=0, dtype=dtype)
    A = np.zeros((C, C), dtype=dtype)
    M = np.zeros((C, C), dtype=dtype)
    nb = (C + block - 1) // block
    for a in range(nb):
        ra = slice(a * block, min(C, (a + 1) * block))
        n = a * block
        row_k = K[ra] * np.exp(G[ra] - G[n])
        row_q = Q[ra] * np.exp(G[ra] - G[n])
        for b in range(a):
            rb = slice(b * block, (b + 1) * block)
            col = K[rb] * np.exp(G[n] - G[rb])
            A[ra, rb] = (row_k @ col.T) * beta[ra, None]
            M[ra, rb] = row_q @ col.T
        for i in range(ra.start, ra.stop):
            for j in range(ra.start, i + 1):
                dec = np.exp(G[i] - G[j])
                M[i, j] = np.dot(Q[i] * dec, K[j])
                if j < i:
                    A[i, j] = beta[i] * np.dot(K[i] * dec, K[j])
    return A, M
