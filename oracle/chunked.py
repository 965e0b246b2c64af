"""Chunked fp64 form of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

The per-chunk algorithm of "Linear Attention, Visualized" (snowchord.com),
section "Gated DeltaNet (GDN)" -> "Complete per-chunk algorithm" for the scalar
gate and section "Reuse GLA and GDN" -> "Complete per-chunk algorithm" for the
channel-wise (KDA) gate, written in that page's own notation: row vectors, state
S_row in R^{d_k x d_v} with o = q S_row.  The library's column-convention state
is the transpose, S = S_row^T in R^{d_v x d_k}; the conversion happens only at
the function boundary.

Decay products are formed literally as products of the per-token decays
a_s = exp(g_s) (lambda[i:j] = prod_{s=i..j} a_s, empty product = 1).  The
triangular system (I + B L) T = B is solved by forward substitution one row at
a time, as the page's section "Solving for U" describes.  Nothing is blocked or
fused; the point is to be checkable against the page by eye.

A ragged last chunk (T not a multiple of C) is simply a shorter chunk: the page
assumes C divides n, and the plainest reading that keeps every chunk size exact
is that the algorithm applies unchanged to a chunk of any length.
"""
from __future__ import annotations

import numpy as np


def _decay_products(a: np.ndarray):
    """lam(i, j) = prod_{s=i..j} a[s-1] for 1-based i, j (identity when i > j).

    ``a`` is [C] (scalar gate) or [C, d_k] (channel gate)."""
    ones = np.ones(a.shape[1:], dtype=np.float64)

    def lam(i: int, j: int):
        if i > j:
            return ones.copy() if a.ndim > 1 else 1.0
        return np.prod(a[i - 1:j], axis=0)

    return lam


def forward_substitution(A: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Solve A X = R for unit-lower-triangular A, row by row."""
    n = A.shape[0]
    X = np.zeros_like(R, dtype=np.float64)
    for t in range(n):
        X[t] = R[t] - A[t, :t] @ X[:t]
    return X


def chunk_transform(K: np.ndarray, g: np.ndarray, beta: np.ndarray):
    """Per-chunk quantities of the page's algorithm (row convention).

    K [C, d_k]; g [C] or [C, d_k] (log-decay); beta [C].
    Returns dict with T, L, decayed keys K_left (rows lam[1:l] k_l) and
    K_right (rows lam[l+1:C] k_l), lam_C (= lam[1:C]) and the lam function.
    """
    K = np.asarray(K, dtype=np.float64)
    a = np.exp(np.asarray(g, dtype=np.float64))
    beta = np.asarray(beta, dtype=np.float64)
    C = K.shape[0]
    lam = _decay_products(a)
    channel = a.ndim == 2
    L = np.zeros((C, C))
    for l in range(1, C + 1):
        for m in range(1, l):
            if channel:
                L[l - 1, m - 1] = K[l - 1] @ (lam(m + 1, l) * K[m - 1])
            else:
                L[l - 1, m - 1] = lam(m + 1, l) * (K[l - 1] @ K[m - 1])
    Bm = np.diag(beta)
    T = forward_substitution(np.eye(C) + Bm @ L, Bm)
    K_left = np.stack([lam(1, l) * K[l - 1] for l in range(1, C + 1)]) if C else K.copy()
    K_right = np.stack([lam(l + 1, C) * K[l - 1] for l in range(1, C + 1)]) if C else K.copy()
    return {"T": T, "L": L, "K_left": K_left, "K_right": K_right, "lam_C": lam(1, C), "lam": lam}


def chunk_scores(Q: np.ndarray, K: np.ndarray, g: np.ndarray):
    """The chunk's local score matrix and decayed queries (row convention).

    A[l, m] = q_l (lam[m+1:l] (.) k_m)^T for m <= l (zero above the diagonal), and Q_left
    with rows lam[1:l] (.) q_l.  Q, K [C, d_k]; g [C] or [C, d_k]."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    lam = _decay_products(np.exp(np.asarray(g, dtype=np.float64)))
    C = Q.shape[0]
    channel = np.ndim(g) == 2
    Q_left = np.stack([lam(1, l) * Q[l - 1] for l in range(1, C + 1)])
    A = np.zeros((C, C))
    for l in range(1, C + 1):
        for m in range(1, l + 1):
            if channel:
                A[l - 1, m - 1] = Q[l - 1] @ (lam(m + 1, l) * K[m - 1])
            else:
                A[l - 1, m - 1] = lam(m + 1, l) * (Q[l - 1] @ K[m - 1])
    return A, Q_left


def _one_chunk(Q, K, V, g, beta, S_row):
    """Advance S_row over one chunk; returns (O [C, d_v], S_row_next)."""
    V = np.asarray(V, dtype=np.float64)
    tr = chunk_transform(K, g, beta)
    T = tr["T"]
    channel = np.ndim(g) == 2
    A, Q_left = chunk_scores(Q, K, g)
    U = T @ V
    W_left = T @ tr["K_left"]
    Z = U - W_left @ S_row
    O = Q_left @ S_row + A @ Z
    if channel:
        S_next = tr["lam_C"][:, None] * S_row + tr["K_right"].T @ Z
    else:
        S_next = tr["lam_C"] * S_row + tr["K_right"].T @ Z
    return O, S_next


def chunked_forward(q, k, v, g, beta, S0=None, C: int = 64):
    """Chunked algorithm over [B,H,T,...] inputs (same layout as the recurrence
    oracle).  Returns (o [B,H,T,d_v], S_T [B,H,d_v,d_k]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = np.shape(v)[-1]
    o = np.zeros((B, H, T, dv))
    S_out = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            S_row = np.zeros((dk, dv)) if S0 is None else np.asarray(S0[b, h], dtype=np.float64).T.copy()
            for start in range(0, T, C):
                end = min(start + C, T)
                O, S_row = _one_chunk(q[b, h, start:end], k[b, h, start:end], v[b, h, start:end],
                                      g[b, h, start:end], beta[b, h, start:end], S_row)
                o[b, h, start:end] = O
            S_out[b, h] = S_row.T
    return o, S_out
