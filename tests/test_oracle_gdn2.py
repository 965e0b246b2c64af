"""Pins for the Gated DeltaNet-2 oracle (runs without a GPU).

``oracle.gdn2_forward`` follows "Gated DeltaNet-2, and the gate that was doing two jobs",
section 2: S_t = (I - k e^T) D S_{t-1} + k z^T (row notation) with e = b (.) k (erase gate b
on the key side) and z = w (.) v (write gate w on the value side).  The checks do not
reuse it:

* the page's collapse: b = w = beta (the same scalar on every channel) is KDA, computed by
  the separately written ``oracle.recurrent_forward`` with the channel gate, and with a
  uniform decay as well it is Gated DeltaNet;
* b = 0 (no erase): the state is a decayed sum of writes, closed form;
* one-hot keys: the erase gate scales exactly one decayed row of the page's state, closed
  form per token;
* b = 1, w = 0, unit keys, no decay: each token is the projection I - k k^T, so repeating a
  token changes nothing;
* the page's formula as dense matrices on tiny inputs (non-unit keys, gates up to 2).

``test_gdn2_planted_mistakes_fail_a_pin`` runs the pins against a plain Python GDN-2
recurrence with one plausible mistake planted at a time.
"""
import numpy as np
import pytest

import oracle

TOL = 1e-12


def f32(x):
    return None if x is None else np.asarray(x, dtype=np.float32).astype(np.float64)


def gdn2_inputs(seed, B=1, H=2, T=7, dk=5, dv=3, unit_k=False, b_range=(0.0, 1.0), w_range=(0.0, 1.0),
                g_range=(-0.7, -0.01), s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, dv))
    g = r.uniform(*g_range, size=(B, H, T, dk))
    b = r.uniform(*b_range, size=(B, H, T, dk))
    w = r.uniform(*w_range, size=(B, H, T, dv))
    S0 = r.standard_normal((B, H, dv, dk)) * 0.5 if s0 else None
    return dict(q=f32(q), k=f32(k), v=f32(v), g=f32(g), b=f32(b), w=f32(w), S0=f32(S0))


def scale(*xs):
    return max(1.0, *[float(np.max(np.abs(x))) for x in xs if x is not None])


# ----------------------------------------------------------------------------- pins
def pin_collapse_to_kda(forward):
    """b = w = beta_t (one scalar per token on every channel) is KDA."""
    x = gdn2_inputs(1, T=9, dk=6, dv=4, unit_k=True)
    beta = f32(np.random.default_rng(2).uniform(0.0, 1.0, size=x["q"].shape[:3]))
    x["b"] = np.repeat(beta[..., None], x["k"].shape[-1], axis=-1)
    x["w"] = np.repeat(beta[..., None], x["v"].shape[-1], axis=-1)
    o, S = forward(**x)
    o2, S2 = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], beta, x["S0"])
    return max(np.max(np.abs(o - o2)), np.max(np.abs(S - S2))) / scale(o2, S2)


def pin_collapse_to_gdn(forward):
    """... and with the same decay on every channel, Gated DeltaNet (scalar gate)."""
    x = gdn2_inputs(3, T=8, dk=5, dv=6)
    r = np.random.default_rng(4)
    beta = f32(r.uniform(0.0, 1.5, size=x["q"].shape[:3]))
    g = f32(r.uniform(-0.5, 0.0, size=x["q"].shape[:3]))
    x["g"] = np.repeat(g[..., None], 5, axis=-1)
    x["b"] = np.repeat(beta[..., None], 5, axis=-1)
    x["w"] = np.repeat(beta[..., None], 6, axis=-1)
    o, S = forward(**x)
    o2, S2 = oracle.recurrent_forward(x["q"], x["k"], x["v"], g, beta, x["S0"])
    return max(np.max(np.abs(o - o2)), np.max(np.abs(S - S2))) / scale(o2, S2)


def pin_no_erase(forward):
    """b = 0: P_t = D_t P_{t-1} + k_t z_t^T, so S_T = S_0 prod D + sum_t z_t (k_t (.) prod_{s>t} a_s)^T
    and o_t = S_t q_t (column convention)."""
    x = gdn2_inputs(5, T=6, b_range=(0.0, 0.0), w_range=(0.0, 2.0))
    o, S = forward(**x)
    B, H, T, dk = x["q"].shape
    errs = []
    for bb in range(B):
        for h in range(H):
            for t in range(T):
                cum = np.exp(np.sum(x["g"][bb, h, :t + 1], axis=0))                  # prod_{s<=t} a_s
                St = x["S0"][bb, h] * cum[None, :]
                for m in range(t + 1):
                    dec = np.exp(np.sum(x["g"][bb, h, m + 1:t + 1], axis=0))         # prod_{m<s<=t} a_s
                    St = St + np.outer(x["w"][bb, h, m] * x["v"][bb, h, m], x["k"][bb, h, m] * dec)
                errs.append(np.max(np.abs(o[bb, h, t] - St @ x["q"][bb, h, t])))
            errs.append(np.max(np.abs(S[bb, h] - St)))
    return max(errs) / scale(o, S)


def pin_one_hot_keys(forward):
    """k_t = e_i: the page's row i becomes (1 - b_i) a_i P_i + w (.) v, every other row only
    decays -- the erase acts on the key side through b_i alone, the write through w alone."""
    dk, dv, T = 4, 3, 6
    x = gdn2_inputs(6, H=1, T=T, dk=dk, dv=dv, b_range=(0.0, 1.0), w_range=(0.0, 1.0))
    idx = np.random.default_rng(7).integers(0, dk, size=T)
    x["k"] = np.zeros_like(x["k"])
    x["k"][0, 0, np.arange(T), idx] = 1.0
    o, S = forward(**x)
    P = x["S0"][0, 0].T.copy()                                  # page state, rows = key channels
    errs = []
    for t in range(T):
        a = np.exp(x["g"][0, 0, t])
        P = a[:, None] * P
        i = idx[t]
        P[i] = (1.0 - x["b"][0, 0, t, i]) * P[i] + x["w"][0, 0, t] * x["v"][0, 0, t]
        errs.append(np.max(np.abs(o[0, 0, t] - x["q"][0, 0, t] @ P)))
    errs.append(np.max(np.abs(S[0, 0] - P.T)))
    return max(errs) / scale(o, S)


def pin_projection_idempotent(forward):
    """b = 1, w = 0, unit keys, a = 1: each token applies the projection I - k k^T; a token
    followed by itself equals the token once, and the state loses its component along k."""
    dk, dv = 8, 3
    x = gdn2_inputs(8, H=1, T=1, dk=dk, dv=dv, b_range=(1.0, 1.0), w_range=(0.0, 0.0), g_range=(0.0, 0.0))
    r = np.random.default_rng(9)
    k = np.zeros(dk)
    k[r.choice(dk, size=4, replace=False)] = r.choice([-0.5, 0.5], size=4)   # exactly unit norm
    x["k"][0, 0, 0] = k
    x2 = {key: (val if key == "S0" else np.concatenate([val, val], axis=2)) for key, val in x.items()}
    _, S1 = forward(**x)
    _, S2 = forward(**x2)
    moved = np.max(np.abs(S1 - x["S0"]))
    return (max(np.max(np.abs(S1 - S2)), np.max(np.abs(S1[0, 0] @ k))) / scale(S1)
            + (0.0 if moved > 1e-3 else 1.0))


def pin_dense_formula(forward):
    """The page's update as dense matrices, P_t = (I - k e^T) D P + k z^T, row notation."""
    x = gdn2_inputs(10, T=5, dk=4, dv=3, b_range=(0.0, 2.0), w_range=(0.0, 2.0))
    o, S = forward(**x)
    errs = []
    for bb in range(o.shape[0]):
        for h in range(o.shape[1]):
            P = x["S0"][bb, h].T.copy()
            for t in range(x["q"].shape[2]):
                k = x["k"][bb, h, t][:, None]
                e = (x["b"][bb, h, t] * x["k"][bb, h, t])[:, None]
                z = (x["w"][bb, h, t] * x["v"][bb, h, t])[:, None]
                D = np.diag(np.exp(x["g"][bb, h, t]))
                P = (np.eye(4) - k @ e.T) @ D @ P + k @ z.T
                errs.append(np.max(np.abs(o[bb, h, t] - x["q"][bb, h, t] @ P)))
            errs.append(np.max(np.abs(S[bb, h] - P.T)))
    return max(errs) / scale(o, S)


def _all_pins(forward):
    with np.errstate(all="ignore"):
        return {"kda": pin_collapse_to_kda(forward), "gdn": pin_collapse_to_gdn(forward),
                "no_erase": pin_no_erase(forward), "one_hot": pin_one_hot_keys(forward),
                "projection": pin_projection_idempotent(forward), "dense": pin_dense_formula(forward)}


def test_gdn2_oracle_passes_every_pin():
    res = _all_pins(oracle.gdn2_forward)
    assert all(val < TOL for val in res.values()), res


@pytest.mark.parametrize("C", [1, 3, 64])
def test_gdn2_chunk_form_passes_every_pin(C):
    """The chunkwise form (``oracle.gdn2_chunked_forward``: the page's WY paragraph, one
    triangular solve for the erase and the write side) meets the same pins."""
    res = _all_pins(lambda **x: oracle.gdn2_chunked_forward(**x, C=C))
    assert all(val < 1e-11 for val in res.values()), res


@pytest.mark.parametrize("C", [1, 2, 4, 16, 64, 150])
def test_gdn2_chunk_form_equals_recurrence(C):
    """Every chunk size gives the token recurrence; T = 150 leaves a ragged tail."""
    x = gdn2_inputs(31, B=1, H=2, T=150, dk=8, dv=6, g_range=(-0.3, -0.001))
    o1, S1 = oracle.gdn2_forward(**x)
    o2, S2 = oracle.gdn2_chunked_forward(**x, C=C)
    assert np.max(np.abs(o1 - o2)) / scale(o1) < 1e-11
    assert np.max(np.abs(S1 - S2)) / scale(S1) < 1e-11


def test_gdn2_empty_sequence_returns_initial_state():
    x = gdn2_inputs(11, T=0)
    o, S = oracle.gdn2_forward(**x)
    assert o.shape == (1, 2, 0, 3) and np.array_equal(S, x["S0"])


def test_gdn2_batches_are_independent():
    x = gdn2_inputs(12, B=2, H=3, T=5)
    o, S = oracle.gdn2_forward(**x)
    one = {key: val[1:2, 2:3] for key, val in x.items()}
    o1, S1 = oracle.gdn2_forward(**one)
    assert np.array_equal(o[1:2, 2:3], o1) and np.array_equal(S[1:2, 2:3], S1)


# ----------------------------------------------------------------------------- planted mistakes
def _python_gdn2(erase_along_k=False, write_along_e=False, gate_swap=False, undecayed_read=False,
                 read_before_write=False, decay_after=False):
    """Plain Python GDN-2 (column convention) with switchable mistakes."""
    def forward(q, k, v, g, b, w, S0=None):
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((B, H, T, dv))
        Sout = np.zeros((B, H, dv, dk))
        for bb in range(B):
            for h in range(H):
                S = np.zeros((dv, dk)) if S0 is None else S0[bb, h].copy()
                for t in range(T):
                    kk, vv, a = k[bb, h, t], v[bb, h, t], np.exp(g[bb, h, t])
                    if gate_swap:   # key gate used on the value side and vice versa (sizes differ:
                        bq = np.resize(w[bb, h, t], dk)
                        wq = np.resize(b[bb, h, t], dv)   # take what fits)
                    else:
                        bq, wq = b[bb, h, t], w[bb, h, t]
                    e = kk if erase_along_k else bq * kk
                    Sd = S * a[None, :]
                    p = (S if undecayed_read else Sd) @ e
                    u = wq * vv - p
                    S = (S if decay_after else Sd) + np.outer(u, e if write_along_e else kk)
                    if decay_after:
                        S = S * a[None, :]
                    if read_before_write:
                        o[bb, h, t] = Sd @ q[bb, h, t]
                    else:
                        o[bb, h, t] = S @ q[bb, h, t]
                Sout[bb, h] = S
        return o, Sout
    return forward


MUTANTS = {
    "erase_along_k_not_e": _python_gdn2(erase_along_k=True),
    "write_along_e_not_k": _python_gdn2(write_along_e=True),
    "gates_swapped": _python_gdn2(gate_swap=True),
    "read_undecayed_state": _python_gdn2(undecayed_read=True),
    "read_before_write": _python_gdn2(read_before_write=True),
    "decay_after_update": _python_gdn2(decay_after=True),
}


def test_gdn2_python_recurrence_passes_pins():
    res = _all_pins(_python_gdn2())
    assert all(val < 1e-10 for val in res.values()), res


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_gdn2_planted_mistakes_fail_a_pin(mutant):
    res = _all_pins(MUTANTS[mutant])
    failed = [key for key, val in res.items() if not (val < 1e-8)]
    assert failed, f"mutant {mutant} passed every pin: {res}"
