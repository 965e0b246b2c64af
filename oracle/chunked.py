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


def gdn2_chunk_transform(K: np.ndarray, E: np.ndarray, g: np.ndarray):
    """Per-chunk quantities of Gated DeltaNet-2 (row convention).

    "Gated DeltaNet-2, and the gate that was doing two jobs" (aigenapps.com), section 2, the
    paragraph on the chunkwise WY representation: with the channel decay normalised out of
    the chunk, the write direction is k_l scaled by the inverse decay and the erase direction
    e_l = b_l (.) k_l by the decay, M = tril(E~ K~^T, -1), and one triangular solve with
    (I + M) serves both right-hand sides.  In terms of the decay products,
    M[l, m] = e_l (lam[m+1:l] (.) k_m)^T for m < l.

    K, E [C, d_k]; g [C, d_k].  Returns dict with M, T_inv = (I + M)^{-1}, E_left (rows
    lam[1:l] (.) e_l), K_right (rows lam[l+1:C] (.) k_l), lam_C and the lam function.
    """
    K = np.asarray(K, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    lam = _decay_products(np.exp(np.asarray(g, dtype=np.float64)))
    C = K.shape[0]
    M = np.zeros((C, C))
    for l in range(1, C + 1):
        for m in range(1, l):
            M[l - 1, m - 1] = E[l - 1] @ (lam(m + 1, l) * K[m - 1])
    T_inv = forward_substitution(np.eye(C) + M, np.eye(C))
    E_left = np.stack([lam(1, l) * E[l - 1] for l in range(1, C + 1)])
    K_right = np.stack([lam(l + 1, C) * K[l - 1] for l in range(1, C + 1)])
    return {"M": M, "T_inv": T_inv, "E_left": E_left, "K_right": K_right, "lam_C": lam(1, C), "lam": lam}


def _gdn2_one_chunk(Q, K, V, g, b, w, S_row):
    """Advance S_row (d_k x d_v) over one Gated DeltaNet-2 chunk; returns (O, S_row_next).

    The erase side Y = (I + M)^{-1} E_left and the write side U_w = (I + M)^{-1} Z come from
    one solve; the corrections are U = U_w - Y S_row; the output is the decayed read of the
    chunk-start state plus the local scores times U, and the state moves by the chunk's
    total decay plus K_right^T U."""
    K = np.asarray(K, dtype=np.float64)
    E = np.asarray(b, dtype=np.float64) * K
    Z = np.asarray(w, dtype=np.float64) * np.asarray(V, dtype=np.float64)
    tr = gdn2_chunk_transform(K, E, g)
    C = K.shape[0]
    rhs = np.concatenate([tr["E_left"], Z], axis=1)
    sol = forward_substitution(np.eye(C) + tr["M"], rhs)
    Y, U_w = sol[:, :K.shape[1]], sol[:, K.shape[1]:]
    U = U_w - Y @ S_row
    A, Q_left = chunk_scores(Q, K, g)
    O = Q_left @ S_row + A @ U
    S_next = tr["lam_C"][:, None] * S_row + tr["K_right"].T @ U
    return O, S_next


def gdn2_chunked_forward(q, k, v, g, b, w, S0=None, C: int = 64):
    """Chunked Gated DeltaNet-2 over [B,H,T,...] inputs (the layout of oracle.gdn2_forward).
    Returns (o [B,H,T,d_v], S_T [B,H,d_v,d_k]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = np.shape(v)[-1]
    o = np.zeros((B, H, T, dv))
    S_out = np.zeros((B, H, dv, dk))
    for bb in range(B):
        for h in range(H):
            S_row = np.zeros((dk, dv)) if S0 is None else np.asarray(S0[bb, h], dtype=np.float64).T.copy()
            for start in range(0, T, C):
                end = min(start + C, T)
                sl = slice(start, end)
                O, S_row = _gdn2_one_chunk(q[bb, h, sl], k[bb, h, sl], v[bb, h, sl], g[bb, h, sl], b[bb, h, sl],
                                           w[bb, h, sl], S_row)
                o[bb, h, sl] = O
            S_out[bb, h] = S_row.T
    return o, S_out
