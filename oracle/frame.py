"""Frame-level implicit delta-rule update -- TEST INFRASTRUCTURE ONLY, fp64 numpy.

Source: the video delta-rule post (haoyizhu.site, "video-delta-rule"), section "A Different
Route" and the remarks that follow it (the implicit step, its Cholesky solve, the frame-level
forget gate and the writing-strength scale).  Tokens come in frames
of n; there is no order inside a frame.  Column convention, state S in R^{d_v x d_k}:

    G_t = K_t^T Gamma_t K_t        (d_k x d_k, symmetric positive semidefinite: the erasure)
    C_t = V_t^T Gamma_t K_t        (d_v x d_k: the write)
    S_t (I + G_t) = S_{t-1} D_t + C_t        (one implicit, backward-Euler gradient step)
    o_{t,i} = S_t q_{t,i}          for every token i of frame t (all read the same S_t)

with Gamma_t = diag(gamma_{t,1..n}) the writing strengths (gamma >= 0) and D_t the frame's
forget gate, applied to the old state before the step (a scalar a_t or one value per key
channel, D_t = Diag(a_t)); the library takes its log, g_t = log a_t.  The post writes the
solve as one Cholesky factorisation of I + G_t followed by one solve; that is what
``frame_forward`` does, step by step, with library primitives (Cholesky, triangular solves,
matrix products).

Reading taken where the page's formula did not survive: the forget gate multiplies S_{t-1}
before C_t is added ("the role of alpha_t is to decay the old state as a whole before taking
this step").  Frames are consecutive groups of ``frame_len`` tokens; a last, shorter frame
holds the remaining tokens.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import cholesky, solve_triangular


def frame_forward(q, k, v, gamma, g, frame_len: int, S0=None):
    """q, k [B,H,T,d_k]; v [B,H,T,d_v]; gamma [B,H,T] (>= 0); g [B,H,F] (scalar gate) or
    [B,H,F,d_k] (per key channel), F = ceil(T / frame_len); S0 [B,H,d_v,d_k] or None.
    Returns (o [B,H,T,d_v], S_F [B,H,d_v,d_k]) in float64."""
    q, k, v, gamma, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, gamma, g))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    n = int(frame_len)
    assert n >= 1
    F = (T + n - 1) // n
    assert g.shape[:3] == (B, H, F) and g.ndim in (3, 4)
    o = np.zeros((B, H, T, dv))
    S_out = np.zeros((B, H, dv, dk))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for f in range(F):
                sl = slice(f * n, min(T, (f + 1) * n))
                K, V, Q, gm = k[b, h, sl], v[b, h, sl], q[b, h, sl], gamma[b, h, sl]
                a = np.exp(g[b, h, f])
                G = K.T @ (gm[:, None] * K)               # erasure
                C = V.T @ (gm[:, None] * K)               # write
                rhs = S * a + C                           # decayed old state (columns scaled by D) + write
                L = cholesky(eye + G, lower=True)         # I + G = L L^T
                # S (I + G) = rhs  <=>  (I + G) S^T = rhs^T: forward then backward substitution
                Y = solve_triangular(L, rhs.T, lower=True)
                S = solve_triangular(L.T, Y, lower=False).T
                o[b, h, sl] = Q @ S.T
            S_out[b, h] = S
    return o, S_out
