"""fp32 models of how the prefill's prep evaluates the per-key A and M diagonal blocks.

[LA-Infra] appendix "附1. chunk内 A和M 的计算" forms e^{G_i - G_j} per key channel. Splitting it
at a reference point n, e^{G_i - G_n} e^{G_n - G_j}, keeps both exponents <= 0 only when
j <= n <= i, which holds for the off-diagonal 16x16 blocks with n = the row block's first
token. Inside a diagonal block (n <= j) the key-side factor e^{G_n - G_j} is >= 1.

These CPU models mirror the kernel's fp32 arithmetic (exponentials in fp32, denormal
results flushed to zero as the hardware does):
  - `split_at_block_start`: the reference-point split applied to the diagonal block as
    well, what the prep did before. It must give non-finite kept entries once a block's
    decay passes fp32's range (g = -6 everywhere: 90 nats over 15 steps; a g = -100 token).
  - `kernel_diag_block`: what the prep does now. The split is kept while the block's
    cumulative decay stays within DIAG_SPAN nats (every factor then sits inside the normal
    range); otherwise the block is computed entry by entry with the mask before the
    exponential, so every kept entry uses e^{G_i - G_j} <= 1.
Both are compared with the fp64 definition of the same entries.
"""
import numpy as np
import pytest

DIAG_SPAN = 60.0
FLT_MIN = np.float32(1.1754944e-38)


def _ftz(x):
    x = np.asarray(x, dtype=np.float32).copy()
    x[np.abs(x) < FLT_MIN] = 0.0
    return x


def _exp32(x):
    with np.errstate(over="ignore", under="ignore"):
        return _ftz(np.exp(np.asarray(x, dtype=np.float32)))


def diag_block_fp64(K, Q, G, rows):
    """A (strictly lower, without beta) and M (lower incl. diagonal) entries of the block:
    sum_c k_i[c] k_j[c] e^{G_i[c] - G_j[c]} and sum_c q_i[c] k_j[c] e^{G_i[c] - G_j[c]},
    indexed [i, j] with i, j local to the block; zero where not kept."""
    K, Q, G = (np.asarray(z, dtype=np.float64) for z in (K, Q, G))
    n = len(rows)
    A, M = np.zeros((n, n)), np.zeros((n, n))
    for a, i in enumerate(rows):
        for b, j in enumerate(rows):
            if j > i:
                continue
            dec = np.exp(G[i] - G[j])
            M[a, b] = np.dot(Q[i] * dec, K[j])
            if j < i:
                A[a, b] = np.dot(K[i] * dec, K[j])
    return A, M


def split_at_block_start(K, Q, G, rows):
    """fp32 split with n = rows[0] for the diagonal block; entries outside the kept part are
    zeroed after the product, as the kernel's output masks do."""
    K, Q, G = (np.asarray(z, dtype=np.float32) for z in (K, Q, G))
    n0 = rows[0]
    fj = _exp32(G[n0] - G[rows])          # key side, >= 1
    fi = _exp32(G[rows] - G[n0])          # row side, <= 1
    with np.errstate(over="ignore", invalid="ignore"):
        kj = _ftz(K[rows] * fj)
        ki = _ftz(K[rows] * fi)
        qi = _ftz(Q[rows] * fi)
        A = (ki @ kj.T).astype(np.float32)
        M = (qi @ kj.T).astype(np.float32)
    keepA = np.tril(np.ones_like(A, dtype=bool), -1)
    keepM = np.tril(np.ones_like(M, dtype=bool))
    return np.where(keepA, A, 0.0), np.where(keepM, M, 0.0), keepA, keepM


def kernel_diag_block(K, Q, G, rows):
    """The prep's current diagonal-block evaluation (fp32 model)."""
    G32 = np.asarray(G, dtype=np.float32)
    span = np.max(G32[rows[0]] - G32[rows[-1]])
    if span <= DIAG_SPAN:
        A, M, _, _ = split_at_block_start(K, Q, G, rows)
        return A, M, "split"
    K, Q = (np.asarray(z, dtype=np.float32) for z in (K, Q))
    n = len(rows)
    A, M = np.zeros((n, n), np.float32), np.zeros((n, n), np.float32)
    for a, i in enumerate(rows):
        for b, j in enumerate(rows):
            # mask before the exponential: only j <= i forms e^{G_i - G_j}
            t = K[j] * _exp32(G32[i] - G32[j]) if j <= i else np.zeros_like(K[j])
            M[a, b] = np.float32(np.dot(Q[i], t))
            if j < i:
                A[a, b] = np.float32(np.dot(K[i], t))
    return A, M, "direct"


def _inputs(kind, seed=0, T=64, dk=128):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T, dk))
    Q = rng.standard_normal((T, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q /= np.linalg.norm(Q, axis=1, keepdims=True)
    K, Q = K.astype(np.float32), Q.astype(np.float32)
    if kind == "minus6":
        g = np.full((T, dk), -6.0)
    elif kind == "hard_forget":
        g = np.log(1.0 / (1.0 + np.exp(-(rng.standard_normal((T, dk)) + 3.0))))
        g[5] = -100.0
        g[37] = -100.0
    elif kind == "uniform30":
        g = -30.0 * rng.random((T, dk))
    elif kind == "workload":  # logsigmoid(randn + 3), the KDA workload's gates
        g = np.log(1.0 / (1.0 + np.exp(-(rng.standard_normal((T, dk)) + 3.0))))
    elif kind == "edge":      # just inside the split's range: 15 steps of -3.95
        g = np.full((T, dk), -3.95)
    else:
        raise ValueError(kind)
    G = np.cumsum(g.astype(np.float32), axis=0, dtype=np.float32)
    return K, Q, G


def _blocks(T=64):
    return [list(range(b, b + 16)) for b in range(0, T, 16)]


@pytest.mark.parametrize("kind", ["minus6", "hard_forget"])
def test_split_at_block_start_breaks(kind):
    """The former evaluation gives non-finite kept entries (inf * 0) at these gates."""
    K, Q, G = _inputs(kind)
    bad = 0
    for rows in _blocks():
        A, M, keepA, keepM = split_at_block_start(K, Q, G, rows)
        bad += int((~np.isfinite(A[keepA])).sum() + (~np.isfinite(M[keepM])).sum())
    assert bad > 0


@pytest.mark.parametrize("kind", ["minus6", "hard_forget", "uniform30", "workload", "edge"])
def test_kernel_scheme_finite_and_exact(kind):
    """The current evaluation is finite and matches the fp64 entries to fp32 rounding, for
    strong, abrupt and ordinary gates alike; the strong kinds take the direct path."""
    K, Q, G = _inputs(kind)
    paths = set()
    for rows in _blocks():
        A, M, path = kernel_diag_block(K, Q, G, rows)
        paths.add(path)
        A_ref, M_ref = diag_block_fp64(K, Q, G, rows)
        assert np.isfinite(A).all() and np.isfinite(M).all()
        scale = max(1.0, np.abs(M_ref).max())
        assert np.abs(A - A_ref).max() <= 1e-5 * scale
        assert np.abs(M - M_ref).max() <= 1e-5 * scale
    if kind in ("minus6", "uniform30"):
        assert paths == {"direct"}
    if kind in ("workload", "edge"):
        assert paths == {"split"}


def test_split_range_bound():
    """Inside DIAG_SPAN both split factors are normal fp32 numbers (and so finite bf16
    operands): e^{60} < FLT_MAX and e^{-60} > FLT_MIN."""
    assert np.isfinite(np.float32(np.exp(DIAG_SPAN)))
    assert np.float32(np.exp(-DIAG_SPAN)) > FLT_MIN
