"""Pins for the frame-level implicit update oracle (``oracle.frame.frame_forward``), CPU only.

The checks do not reuse it:

* n = 1: by Sherman-Morrison the implicit step is the delta rule with learning rate
  gamma / (1 + gamma) (the post's single-token case), so it must equal the separately
  written GDN token recurrence with beta = gamma / (1 + gamma) and the same log-decay;
* permuting the tokens inside each frame permutes the outputs the same way and leaves the
  state unchanged (the post's permutation invariance);
* orthonormal keys in a frame: (I + G)^{-1} = I - sum_i gamma_i / (1 + gamma_i) k_i k_i^T,
  i.e. the delta rule over the frame's tokens in any order (closed form by orthogonality);
* gamma = 0: pure decay; and gamma -> large on one token: the state reads v back at k;
* the defining equation S_t (I + G_t) = S_{t-1} D_t + C_t, checked with an independent dense
  solve (numpy.linalg.solve) rather than the oracle's Cholesky route.

``test_frame_planted_mistakes_fail_a_pin`` runs the pins against a plain dense-solve
implementation with one plausible mistake planted at a time.
"""
import numpy as np
import pytest

import oracle
from oracle.frame import frame_forward

TOL = 1e-10


def f32(x):
    return None if x is None else np.asarray(x, dtype=np.float32).astype(np.float64)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def frame_inputs(seed, B=1, H=2, F=3, n=5, dk=6, dv=4, channel=False, gamma_scale=1.0, s0=True):
    r = np.random.default_rng(seed)
    T = F * n
    q = r.standard_normal((B, H, T, dk))
    k = unit(r.standard_normal((B, H, T, dk)))
    v = r.standard_normal((B, H, T, dv))
    gamma = gamma_scale * np.exp(0.5 * r.standard_normal((B, H, T)))
    g = r.uniform(-0.5, -0.01, size=(B, H, F, dk) if channel else (B, H, F))
    S0 = r.standard_normal((B, H, dv, dk)) * 0.5 if s0 else None
    return dict(q=f32(q), k=f32(k), v=f32(v), gamma=f32(gamma), g=f32(g), S0=f32(S0)), n


def scale(*xs):
    return max(1.0, *[float(np.max(np.abs(x))) for x in xs if x is not None])


# ----------------------------------------------------------------------------- pins
def pin_single_token_is_delta_rule(forward):
    x, _ = frame_inputs(1, F=7, n=1, dk=5, dv=3)
    # beta exact in binary (the C recurrence takes float32), gamma = beta / (1 - beta) in fp64
    r = np.random.default_rng(11)
    beta = r.integers(1, 16, size=x["gamma"].shape) / 16.0
    x["gamma"] = beta / (1.0 - beta)
    # keys of exactly unit norm (Sherman-Morrison gives gamma / (1 + gamma ||k||^2))
    k = np.zeros_like(x["k"])
    for row in k.reshape(-1, k.shape[-1]):
        row[r.choice(k.shape[-1], size=4, replace=False)] = r.choice([-0.5, 0.5], size=4)
    x["k"] = k
    o, S = forward(frame_len=1, **x)
    o2, S2 = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], beta, x["S0"])
    return max(np.max(np.abs(o - o2)), np.max(np.abs(S - S2))) / scale(o2, S2)


def pin_permutation_invariance(forward, channel=False):
    x, n = frame_inputs(2, F=3, n=6, dk=5, dv=3, channel=channel)
    o, S = forward(frame_len=n, **x)
    r = np.random.default_rng(3)
    T = x["q"].shape[2]
    perm = np.concatenate([f * n + r.permutation(n) for f in range(T // n)])
    xp = {key: (val[:, :, perm] if key in ("q", "k", "v", "gamma") else val) for key, val in x.items()}
    op, Sp = forward(frame_len=n, **xp)
    return max(np.max(np.abs(op - o[:, :, perm])), np.max(np.abs(Sp - S))) / scale(o, S)


def pin_orthonormal_keys(forward):
    """Frames of n <= d_k orthonormal keys: S_t = (S_{t-1} D + C) (I - sum gamma/(1+gamma) k k^T)."""
    dk, dv, n, F = 6, 3, 4, 3
    x, _ = frame_inputs(4, H=1, F=F, n=n, dk=dk, dv=dv)
    r = np.random.default_rng(5)
    for f in range(F):
        Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
        x["k"][0, 0, f * n:(f + 1) * n] = Qm[:, :n].T
    o, S = forward(frame_len=n, **x)
    St = x["S0"][0, 0].copy()
    errs = []
    for f in range(F):
        sl = slice(f * n, (f + 1) * n)
        K, V, gm = x["k"][0, 0, sl], x["v"][0, 0, sl], x["gamma"][0, 0, sl]
        P = np.eye(dk) - (K.T * (gm / (1.0 + gm))) @ K
        St = (St * np.exp(x["g"][0, 0, f]) + (V.T * gm) @ K) @ P
        errs.append(np.max(np.abs(o[0, 0, sl] - x["q"][0, 0, sl] @ St.T)))
    errs.append(np.max(np.abs(S[0, 0] - St)))
    return max(errs) / scale(o, S)


def pin_no_write_is_pure_decay(forward):
    x, n = frame_inputs(6, F=4, n=3, channel=True)
    x["gamma"] = np.zeros_like(x["gamma"])
    o, S = forward(frame_len=n, **x)
    cum = np.exp(np.cumsum(x["g"], axis=2))                         # [B,H,F,dk]
    S_ref = x["S0"] * cum[:, :, -1][:, :, None, :]
    tok_cum = np.repeat(cum, n, axis=2)                             # per token of each frame
    o_ref = np.einsum("bhvc,bhtc->bhtv", x["S0"], x["q"] * tok_cum)
    return max(np.max(np.abs(o - o_ref)), np.max(np.abs(S - S_ref))) / scale(o_ref, S_ref)


def pin_strong_write_reads_back(forward):
    """One token with gamma = 1e6: S_1 k = v to within 1e-5 (the old content at k is erased)."""
    x, _ = frame_inputs(7, H=1, F=1, n=1, dk=5, dv=3)
    x["gamma"][:] = 1e6
    _, S = forward(frame_len=1, **x)
    return np.max(np.abs(S[0, 0] @ x["k"][0, 0, 0] - x["v"][0, 0, 0])) * 1e-5


def pin_defining_equation(forward, channel=True):
    """S_t (I + G_t) = S_{t-1} D_t + C_t, frame by frame, solved densely with numpy.linalg.solve;
    the outputs read S_t.  A ragged last frame included."""
    x, n = frame_inputs(8, F=3, n=4, dk=5, dv=4, channel=channel)
    T = 10                                                          # frames of 4, 4, 2 tokens
    for key in ("q", "k", "v", "gamma"):
        x[key] = x[key][:, :, :T]
    o, S = forward(frame_len=n, **x)
    errs = []
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            St = x["S0"][b, h].copy()
            for f in range(3):
                sl = slice(f * n, min(T, (f + 1) * n))
                K, V, gm = x["k"][b, h, sl], x["v"][b, h, sl], x["gamma"][b, h, sl]
                A = np.eye(K.shape[1]) + (K.T * gm) @ K
                rhs = St * np.exp(x["g"][b, h, f]) + (V.T * gm) @ K
                St = np.linalg.solve(A.T, rhs.T).T
                errs.append(np.max(np.abs(o[b, h, sl] - x["q"][b, h, sl] @ St.T)))
            errs.append(np.max(np.abs(S[b, h] - St)))
    return max(errs) / scale(o, S)


def _all_pins(forward):
    with np.errstate(all="ignore"):
        try:
            return {"single_token": pin_single_token_is_delta_rule(forward),
                    "perm": pin_permutation_invariance(forward),
                    "perm_channel": pin_permutation_invariance(forward, channel=True),
                    "orthonormal": pin_orthonormal_keys(forward),
                    "no_write": pin_no_write_is_pure_decay(forward),
                    "strong_write": pin_strong_write_reads_back(forward),
                    "equation": pin_defining_equation(forward),
                    "equation_scalar": pin_defining_equation(forward, channel=False)}
        except np.linalg.LinAlgError:
            return {"linalg_error": 1.0}


def test_frame_oracle_passes_every_pin():
    res = _all_pins(frame_forward)
    assert all(val < TOL for val in res.values()), res


def test_frame_empty_sequence_returns_initial_state():
    x, _ = frame_inputs(9, F=1, n=2)
    x = {key: (val[:, :, :0] if key in ("q", "k", "v", "gamma", "g") else val) for key, val in x.items()}
    o, S = frame_forward(frame_len=2, **x)
    assert o.shape[2] == 0 and np.array_equal(S, x["S0"])


# ----------------------------------------------------------------------------- planted mistakes
def _dense(decay_after=False, explicit_step=False, read_old_state=False, gamma_on_erase_only=False,
           transpose_solve=False):
    """Dense-solve frame update with switchable mistakes."""
    def forward(q, k, v, gamma, g, frame_len, S0=None):
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        n = frame_len
        F = (T + n - 1) // n
        o = np.zeros((B, H, T, dv))
        Sout = np.zeros((B, H, dv, dk))
        for b in range(B):
            for h in range(H):
                S = np.zeros((dv, dk)) if S0 is None else S0[b, h].copy()
                for f in range(F):
                    sl = slice(f * n, min(T, (f + 1) * n))
                    K, V, gm = k[b, h, sl], v[b, h, sl], gamma[b, h, sl]
                    a = np.exp(g[b, h, f])
                    G = (K.T * gm) @ K
                    C = V.T @ K if gamma_on_erase_only else (V.T * gm) @ K
                    old = S
                    if explicit_step:
                        S = (S * a) @ (np.eye(dk) - G) + C
                    elif decay_after:
                        S = np.linalg.solve((np.eye(dk) + G).T, (S + C).T).T * a
                    elif transpose_solve:   # only the lower triangle of G kept (not symmetric)
                        S = (S * a + C) @ np.linalg.inv(np.eye(dk) + np.tril(G))
                    else:
                        S = np.linalg.solve((np.eye(dk) + G).T, (S * a + C).T).T
                    o[b, h, sl] = q[b, h, sl] @ (old if read_old_state else S).T
                Sout[b, h] = S
        return o, Sout
    return forward


MUTANTS = {
    "decay_after_solve": _dense(decay_after=True),
    "explicit_euler_step": _dense(explicit_step=True),
    "read_previous_state": _dense(read_old_state=True),
    "write_without_gamma": _dense(gamma_on_erase_only=True),
    "asymmetric_system": _dense(transpose_solve=True),
}


def test_frame_dense_solve_passes_pins():
    res = _all_pins(_dense())
    assert all(val < 1e-9 for val in res.values()), res


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_frame_planted_mistakes_fail_a_pin(mutant):
    res = _all_pins(MUTANTS[mutant])
    failed = [key for key, val in res.items() if not (val < 1e-8)]
    assert failed, f"mutant {mutant} passed every pin: {res}"
