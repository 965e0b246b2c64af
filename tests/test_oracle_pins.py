"""Pins for the CPU oracle (runs without a GPU).

Every check below compares the oracle with something that does not reuse it:
closed forms, limits, an independently coded parallel form, brute-force dense
matrix products, or identities stated on the pages.  Sizes are tiny, fp64,
tolerance 1e-12 (relative to the data's scale) unless noted.

The pins are written as functions of a ``forward`` callable so that
``test_planted_mistakes_fail_a_pin`` can run them against deliberately wrong
CPU recurrences and show that each plausible mistake is caught.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.chunked import chunk_scores, chunk_transform, chunked_forward

TOL = 1e-12
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- inputs
def rand_inputs(seed, B=1, H=2, T=9, dk=5, dv=3, gate="scalar", unit_k=True, beta_range=(0.05, 1.0),
                g_range=(-0.6, -0.01), s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, dv))
    beta = r.uniform(*beta_range, size=(B, H, T))
    gshape = (B, H, T) if gate == "scalar" else (B, H, T, dk)
    g = r.uniform(*g_range, size=gshape)
    S0 = r.standard_normal((B, H, dv, dk)) * 0.5 if s0 else None
    # the oracle takes float32 inputs (exact values handed to the GPU); make the
    # fp64 copies exactly float32-representable so both see identical numbers
    f = lambda x: None if x is None else x.astype(np.float32).astype(np.float64)
    return dict(q=f(q), k=f(k), v=f(v), g=f(g), beta=f(beta), S0=f(S0))


def exact_unit_keys(seed, shape):
    """Keys with exactly unit norm in binary: four entries of +-1/2 at random
    positions (d_k >= 4), so pins that need ||k|| = 1 hold without rounding."""
    r = np.random.default_rng(seed)
    k = np.zeros(shape)
    flat = k.reshape(-1, shape[-1])
    for row in flat:
        idx = r.choice(shape[-1], size=4, replace=False)
        row[idx] = r.choice([-0.5, 0.5], size=4)
    return k


def oracle_forward(q, k, v, g, beta, S0=None):
    return oracle.recurrent_forward(q, k, v, g, beta, S0)


def scale(*xs):
    return max(1.0, *[float(np.max(np.abs(x))) for x in xs if x is not None])


# ----------------------------------------------------------------------------- pins
def pin_p1_beta_zero(forward, gate):
    """P1: beta = 0 leaves only the decay: S_T = S0 * prod(a) and o_t = (decayed S0) q_t."""
    x = rand_inputs(11, gate=gate, dk=5, dv=3)
    x["beta"][:] = 0.0
    o, S = forward(**x)
    a = np.exp(x["g"])
    cum = np.cumprod(a, axis=2)  # prod_{s<=t} a_s (per channel for KDA)
    errs = []
    for b in range(x["q"].shape[0]):
        for h in range(x["q"].shape[1]):
            S0 = x["S0"][b, h]
            for t in range(x["q"].shape[2]):
                if gate == "scalar":
                    ref = cum[b, h, t] * (S0 @ x["q"][b, h, t])
                else:
                    ref = S0 @ (cum[b, h, t] * x["q"][b, h, t])
                errs.append(np.max(np.abs(o[b, h, t] - ref)))
            Sref = S0 * (cum[b, h, -1] if gate == "scalar" else cum[b, h, -1][None, :])
            errs.append(np.max(np.abs(S[b, h] - Sref)))
    return max(errs)


def pin_p2_identity_tokens(forward, gate):
    """P2: g = 0 and beta = 0 is the identity transition; padding with such tokens
    changes neither the state nor the outputs of the real tokens."""
    x = rand_inputs(12, gate=gate)
    y = {kk: (None if vv is None else vv.copy()) for kk, vv in x.items()}
    y["g"][:] = 0.0
    y["beta"][:] = 0.0
    o, S = forward(**y)
    e1 = max(np.max(np.abs(S - y["S0"])),
             np.max(np.abs(o - np.einsum("bhvc,bhtc->bhtv", y["S0"], y["q"]))))
    # pad the real sequence with 5 identity tokens (random q, k, v)
    pad = rand_inputs(13, gate=gate, T=5)
    z = {}
    for key in ("q", "k", "v", "g", "beta"):
        p = pad[key].copy()
        if key in ("g", "beta"):
            p[:] = 0.0
        z[key] = np.concatenate([x[key], p], axis=2)
    o1, S1 = forward(**x)
    o2, S2 = forward(**z, S0=x["S0"])
    T = x["q"].shape[2]
    e2 = max(np.max(np.abs(S1 - S2)), np.max(np.abs(o1 - o2[:, :, :T])))
    return max(e1, e2) / scale(S1, o1)


def deltanet_parallel_form(q, k, v, beta):
    """DeltaNet full-sequence form ("Linear Attention, Visualized", sections
    "The triangular correction system" and "Parallel output"), row convention:
    L = (K K^T) (.) M^-, (I + B L) U = B V, O = (Q K^T (.) M) U."""
    n = q.shape[0]
    M = np.tril(np.ones((n, n)))
    Mm = M - np.eye(n)
    L = (k @ k.T) * Mm
    Bm = np.diag(beta)
    U = np.linalg.solve(np.eye(n) + Bm @ L, Bm @ v)
    return ((q @ k.T) * M) @ U, k.T @ U  # O, S_row = K^T U


def pin_p3_deltanet(forward, dk=6, dv=4):
    """P3: alpha = 1 (g = 0), S0 = 0 reduces to DeltaNet's parallel form (non-unit keys too)."""
    x = rand_inputs(14, T=11, dk=dk, dv=dv, unit_k=False, beta_range=(0.0, 1.5), s0=False)
    x["g"][:] = 0.0
    o, S = forward(**x)
    errs = []
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            O, S_row = deltanet_parallel_form(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["beta"][b, h])
            errs += [np.max(np.abs(o[b, h] - O)), np.max(np.abs(S[b, h] - S_row.T))]
    return max(errs) / scale(o, S)


def _prefix_states(forward, x, gate):
    """States S_0..S_T by running the forward on every prefix."""
    T = x["q"].shape[2]
    states = [x["S0"]]
    for t in range(1, T + 1):
        _, S = forward(**{kk: (vv[:, :, :t] if kk not in ("S0",) else vv) for kk, vv in x.items()})
        states.append(S)
    return states


def pin_p4_beta_one(forward, gate):
    """P4: beta = 1 with unit keys writes exactly: S_t k_t = v_t for every t."""
    x = rand_inputs(15, gate=gate, T=7)
    x["k"] = exact_unit_keys(115, x["k"].shape)
    x["beta"][:] = 1.0
    st = _prefix_states(forward, x, gate)
    errs = []
    for t in range(1, x["q"].shape[2] + 1):
        Sk = np.einsum("bhvc,bhc->bhv", st[t], x["k"][:, :, t - 1])
        errs.append(np.max(np.abs(Sk - x["v"][:, :, t - 1])))
    return max(errs)


def pin_p5_orthonormal_keys(forward, gate):
    """P5: orthonormal keys k_t = e_t (T <= d_k), S0 = 0: the erase term vanishes and
    the output is gated accumulation, o_t = sum_{j<=t} (q_t . (lam[j+1:t] k_j)) beta_j v_j."""
    T, dk, dv = 6, 8, 5
    x = rand_inputs(16, gate=gate, T=T, dk=dk, dv=dv, s0=False)
    x["k"][:] = 0.0
    for t in range(T):
        x["k"][:, :, t, t] = 1.0
    o, S = forward(**x)
    a = np.exp(x["g"])
    ref = np.zeros_like(o)
    Sref = np.zeros_like(S)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            for t in range(T):
                for j in range(t + 1):
                    lam = np.prod(a[b, h, j + 1:t + 1], axis=0)  # decay from j+1 to t
                    w = x["q"][b, h, t] @ (lam * x["k"][b, h, j])
                    ref[b, h, t] += w * x["beta"][b, h, j] * x["v"][b, h, j]
            for j in range(T):
                lam = np.prod(a[b, h, j + 1:T], axis=0)
                Sref[b, h] += x["beta"][b, h, j] * np.outer(x["v"][b, h, j], lam * x["k"][b, h, j])
    return max(np.max(np.abs(o - ref)), np.max(np.abs(S - Sref))) / scale(o, S)


def pin_p6_mix_identity(forward, gate):
    """P6: reading the new state at k_t gives (1 - beta_t n_t) p_t + beta_t n_t v_t with
    n_t = ||k_t||^2 and p_t the prediction from the decayed previous state; for unit keys
    this is the page's (1 - beta_t) p_t + beta_t v_t ("An intuitive example", which also
    names the extra ||k_t||^2 factor for non-unit keys).  Keys here are not unit."""
    x = rand_inputs(17, gate=gate, T=7, beta_range=(0.0, 2.0), unit_k=False)
    st = _prefix_states(forward, x, gate)
    a = np.exp(x["g"])
    errs = []
    for t in range(1, x["q"].shape[2] + 1):
        k = x["k"][:, :, t - 1]
        if gate == "scalar":
            p = a[:, :, t - 1][..., None] * np.einsum("bhvc,bhc->bhv", st[t - 1], k)
        else:
            p = np.einsum("bhvc,bhc->bhv", st[t - 1], a[:, :, t - 1] * k)
        bt = x["beta"][:, :, t - 1][..., None] * np.sum(k * k, axis=-1, keepdims=True)
        ref = (1 - bt) * p + bt * x["v"][:, :, t - 1]
        errs.append(np.max(np.abs(np.einsum("bhvc,bhc->bhv", st[t], k) - ref)))
    return max(errs)


def pin_dense_transition(forward, gate):
    """The update written as dense matrices, S_t = S_{t-1} D_t (I - b k k^T) + b v k^T
    (D_t = a_t I or Diag(a_t)), with non-unit keys, beta up to 2 and d_k != d_v."""
    x = rand_inputs(18, gate=gate, T=6, dk=5, dv=3, unit_k=False, beta_range=(0.0, 2.0))
    o, S = forward(**x)
    a = np.exp(x["g"])
    errs = []
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            St = x["S0"][b, h].copy()
            for t in range(x["q"].shape[2]):
                k = x["k"][b, h, t][:, None]
                v = x["v"][b, h, t][:, None]
                be = x["beta"][b, h, t]
                D = a[b, h, t] * np.eye(k.shape[0]) if gate == "scalar" else np.diag(a[b, h, t])
                St = St @ D @ (np.eye(k.shape[0]) - be * k @ k.T) + be * v @ k.T
                errs.append(np.max(np.abs(o[b, h, t] - St @ x["q"][b, h, t])))
            errs.append(np.max(np.abs(S[b, h] - St)))
    return max(errs) / scale(o, S)


def pin_p11_first_rows(forward):
    """P11: the first three correction rows in closed form (DeltaNet, alpha = 1):
    u1 = b1 v1, u2 = b2 (v2 - (k2.k1) u1), u3 = b3 (v3 - (k3.k1) u1 - (k3.k2) u2);
    S_3 = sum_i u_i k_i^T and o_3 = S_3 q_3."""
    x = rand_inputs(19, B=1, H=1, T=3, dk=4, dv=3, unit_k=False, s0=False)
    x["g"][:] = 0.0
    o, S = forward(**x)
    k, v, q, b = x["k"][0, 0], x["v"][0, 0], x["q"][0, 0], x["beta"][0, 0]
    u1 = b[0] * v[0]
    u2 = b[1] * (v[1] - (k[1] @ k[0]) * u1)
    u3 = b[2] * (v[2] - (k[2] @ k[0]) * u1 - (k[2] @ k[1]) * u2)
    S3 = np.outer(u1, k[0]) + np.outer(u2, k[1]) + np.outer(u3, k[2])
    S1 = np.outer(u1, k[0])
    S2 = S1 + np.outer(u2, k[1])
    e = max(np.max(np.abs(S[0, 0] - S3)), np.max(np.abs(o[0, 0, 2] - S3 @ q[2])),
            np.max(np.abs(o[0, 0, 1] - S2 @ q[1])), np.max(np.abs(o[0, 0, 0] - S1 @ q[0])))
    return e / scale(S3)


def pin_p12_linearity(forward, gate):
    """P12: (o, S_T) is jointly linear in (V, S0) for fixed q, k, g, beta."""
    x = rand_inputs(20, gate=gate)
    y = rand_inputs(21, gate=gate)
    # values on a 2^-8 grid and integer coefficients keep every combination exact in float32
    for d in (x, y):
        d["v"] = np.round(d["v"] * 256) / 256
        d["S0"] = np.round(d["S0"] * 256) / 256
    c1, c2 = 3.0, -2.0
    z = dict(x)
    z["v"] = c1 * x["v"] + c2 * y["v"]
    z["S0"] = c1 * x["S0"] + c2 * y["S0"]
    yy = dict(x)
    yy["v"], yy["S0"] = y["v"], y["S0"]
    o1, S1 = forward(**x)
    o2, S2 = forward(**yy)
    o3, S3 = forward(**z)
    return max(np.max(np.abs(o3 - (c1 * o1 + c2 * o2))), np.max(np.abs(S3 - (c1 * S1 + c2 * S2)))) / scale(o3, S3)


def pin_p13_split(forward, gate):
    """P13: running x[:t0] then x[t0:] from the carried state equals running x."""
    x = rand_inputs(22, gate=gate, T=13)
    o, S = forward(**x)
    errs = []
    for t0 in (1, 4, 8, 12):
        a = {kk: (vv[:, :, :t0] if kk != "S0" else vv) for kk, vv in x.items()}
        oa, Sa = forward(**a)
        b = {kk: vv[:, :, t0:] for kk, vv in x.items() if kk != "S0"}
        ob, Sb = forward(**b, S0=Sa)
        errs += [np.max(np.abs(np.concatenate([oa, ob], axis=2) - o)), np.max(np.abs(Sb - S))]
    return max(errs) / scale(o, S)


def pin_alice_bob(forward):
    """The page's worked example ("An intuitive example"), fixture in tests/golden/alice_bob.json."""
    with open(os.path.join(GOLDEN, "alice_bob.json")) as f:
        ex = json.load(f)
    ka, kb = (np.array(ex["keys"][n]) for n in ("alice", "bob"))
    vs, vh, vo = (np.array(ex["values"][n]) for n in ("school", "home", "office"))
    S0 = np.outer(vs, ka) + np.outer(vh, kb)  # memory holding both associations
    errs = []
    for b in ex["betas"]:
        x = dict(q=ka.reshape(1, 1, 1, -1), k=kb.reshape(1, 1, 1, -1), v=vo.reshape(1, 1, 1, -1),
                 g=np.zeros((1, 1, 1)), beta=np.full((1, 1, 1), b), S0=S0.reshape(1, 1, len(vs), len(ka)))
        o, S = forward(**x)
        errs.append(np.max(np.abs(S[0, 0] @ kb - ((1 - b) * vh + b * vo))))
        errs.append(np.max(np.abs(S[0, 0] @ ka - vs)))  # Alice's read is untouched
        errs.append(np.max(np.abs(o[0, 0, 0] - vs)))      # query at Alice's key
    return max(errs)


GATES = ("scalar", "channel")


# ----------------------------------------------------------------------------- oracle tests
@pytest.mark.parametrize("gate", GATES)
def test_p1_beta_zero(gate):
    assert pin_p1_beta_zero(oracle_forward, gate) < TOL


@pytest.mark.parametrize("gate", GATES)
def test_p2_identity_tokens(gate):
    assert pin_p2_identity_tokens(oracle_forward, gate) < TOL


@pytest.mark.parametrize("dk,dv", [(6, 4), (5, 5), (3, 7)])
def test_p3_deltanet_parallel_form(dk, dv):
    assert pin_p3_deltanet(oracle_forward, dk, dv) < 1e-10


@pytest.mark.parametrize("gate", GATES)
def test_p4_beta_one_exact_write(gate):
    assert pin_p4_beta_one(oracle_forward, gate) < 1e-11


@pytest.mark.parametrize("gate", GATES)
def test_p5_orthonormal_keys(gate):
    assert pin_p5_orthonormal_keys(oracle_forward, gate) < TOL


@pytest.mark.parametrize("gate", GATES)
def test_p6_mix_identity(gate):
    assert pin_p6_mix_identity(oracle_forward, gate) < 1e-11


@pytest.mark.parametrize("gate", GATES)
def test_dense_transition_form(gate):
    assert pin_dense_transition(oracle_forward, gate) < TOL


def test_p11_first_rows():
    assert pin_p11_first_rows(oracle_forward) < TOL


@pytest.mark.parametrize("gate", GATES)
def test_p12_linearity(gate):
    assert pin_p12_linearity(oracle_forward, gate) < TOL


@pytest.mark.parametrize("gate", GATES)
def test_p13_carried_state_split(gate):
    assert pin_p13_split(oracle_forward, gate) < TOL


def test_alice_bob_example():
    assert pin_alice_bob(oracle_forward) < TOL


@pytest.mark.parametrize("gate", GATES)
def test_p7_wy_ut_product(gate):
    """P7: per chunk, the ordered product of transitions equals the WY/UT form
    lam[1:C] - K_right^T T K_left (row convention, "Lemma" + "Compact the transition
    product with WY" + "Use UT..."), and the convolution sum H equals K_right^T T V."""
    x = rand_inputs(23, B=1, H=1, T=8, dk=6, dv=4, gate=gate, unit_k=False, beta_range=(0.0, 1.5))
    K, V, g, beta = x["k"][0, 0], x["v"][0, 0], x["g"][0, 0], x["beta"][0, 0]
    tr = chunk_transform(K, g, beta)
    a = np.exp(g)
    dk = K.shape[1]
    Lam = np.eye(dk)
    H = np.zeros((dk, V.shape[1]))
    for l in range(K.shape[0]):  # row convention: S_l = A_l S_{l-1} + X_l
        D = a[l] * np.eye(dk) if gate == "scalar" else np.diag(a[l])
        A_l = (np.eye(dk) - beta[l] * np.outer(K[l], K[l])) @ D
        Lam = A_l @ Lam
        H = A_l @ H + beta[l] * np.outer(K[l], V[l])
    lamC = tr["lam_C"] * np.eye(dk) if gate == "scalar" else np.diag(tr["lam_C"])
    wy = lamC - tr["K_right"].T @ tr["T"] @ tr["K_left"]
    assert np.max(np.abs(Lam - wy)) < 1e-12
    assert np.max(np.abs(H - tr["K_right"].T @ tr["T"] @ V)) < 1e-12


@pytest.mark.parametrize("gate", GATES)
def test_chunk_quantities_closed_forms(gate):
    """The per-chunk quantities in log space ("Gated DeltaNet (GDN)" and "Reuse GLA and GDN"
    sections: q_left, k_left, k_right and the decay inside the local scores), written with the
    inclusive cumulative log-decay G instead of the oracle's products of e^{g}:
    A[l, m] = sum_c q_lc k_mc e^{G_lc - G_mc} (m <= l), q_left = e^{G} q, k_left = e^{G} k,
    k_right = e^{G_C - G} k, lam_C = e^{G_C}."""
    x = rand_inputs(29, B=1, H=1, T=11, dk=6, dv=3, gate=gate, unit_k=False, g_range=(-0.4, -0.01))
    Q, K, g, beta = x["q"][0, 0], x["k"][0, 0], x["g"][0, 0], x["beta"][0, 0]
    G = np.cumsum(g, axis=0)
    Gc = G if gate == "channel" else G[:, None] * np.ones(K.shape[1])
    C = K.shape[0]
    A_ref = np.zeros((C, C))
    for l in range(C):
        for m in range(l + 1):
            A_ref[l, m] = np.sum(Q[l] * K[m] * np.exp(Gc[l] - Gc[m]))
    A, Q_left = chunk_scores(Q, K, g)
    assert np.max(np.abs(A - A_ref)) / scale(A_ref) < TOL
    assert np.max(np.abs(Q_left - np.exp(Gc) * Q)) / scale(Q) < TOL
    tr = chunk_transform(K, g, beta)
    assert np.max(np.abs(tr["K_left"] - np.exp(Gc) * K)) / scale(K) < TOL
    assert np.max(np.abs(tr["K_right"] - np.exp(Gc[-1] - Gc) * K)) / scale(K) < TOL
    assert np.max(np.abs(np.asarray(tr["lam_C"]) - np.exp(G[-1]))) < TOL


@pytest.mark.parametrize("gate", GATES)
@pytest.mark.parametrize("C", [1, 2, 4, 16, 64, 150])
def test_p8_chunked_equals_recurrence(gate, C):
    """P8: every chunk size gives the exact result ("Cost"); T=150 leaves a ragged tail."""
    x = rand_inputs(24, B=1, H=2, T=150, dk=8, dv=6, gate=gate, g_range=(-0.3, -0.001))
    o1, S1 = oracle_forward(**x)
    o2, S2 = chunked_forward(**x, C=C)
    assert np.max(np.abs(o1 - o2)) / scale(o1) < 1e-11
    assert np.max(np.abs(S1 - S2)) / scale(S1) < 1e-11


def test_p9_kda_uniform_equals_gdn():
    """P9: a channel gate that is the same in every channel is the scalar gate."""
    x = rand_inputs(25, gate="scalar")
    o1, S1 = oracle_forward(**x)
    y = dict(x)
    y["g"] = np.repeat(x["g"][..., None], x["k"].shape[-1], axis=-1)
    o2, S2 = oracle_forward(**y)
    assert np.max(np.abs(o1 - o2)) < TOL and np.max(np.abs(S1 - S2)) < TOL


@pytest.mark.parametrize("gate", GATES)
def test_p10_decode_loop_equals_forward(gate):
    """P10: T decode steps on a resident state equal the forward over the same T tokens."""
    x = rand_inputs(26, B=2, H=3, T=6, gate=gate)
    o, S = oracle_forward(**x)
    St = x["S0"].copy()
    for t in range(x["q"].shape[2]):
        ot, St = oracle.decode_step(x["q"][:, :, t], x["k"][:, :, t], x["v"][:, :, t],
                                    x["g"][:, :, t], x["beta"][:, :, t], St)
        assert np.max(np.abs(ot - o[:, :, t])) < TOL
    assert np.max(np.abs(St - S)) < TOL


def test_empty_sequence_returns_initial_state():
    x = rand_inputs(27, T=0)
    o, S = oracle_forward(**x)
    assert o.shape[2] == 0 and np.array_equal(S, x["S0"])


# ----------------------------------------------------------------------------- pin power
def _python_recurrence(read_before_write=False, undecayed_prediction=False, kda_rows=False,
                       drop_beta_in_prediction=False, decay_after_write=False):
    """A CPU recurrence with one planted mistake, to show the pins catch it."""

    def forward(q, k, v, g, beta, S0=None):
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((B, H, T, dv))
        Sout = np.zeros((B, H, dv, dk))
        for b in range(B):
            for h in range(H):
                S = np.zeros((dv, dk)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
                for t in range(T):
                    a = np.exp(g[b, h, t])
                    kt, vt, qt, bt = k[b, h, t], v[b, h, t], q[b, h, t], beta[b, h, t]
                    if read_before_write:
                        o[b, h, t] = S @ qt
                    if np.ndim(a) == 0:
                        Sd = S * a
                    else:
                        Sd = a[:dv, None] * S if kda_rows else S * a[None, :]
                    p = (S if undecayed_prediction else Sd) @ kt
                    u = bt * vt - p if drop_beta_in_prediction else bt * (vt - p)
                    if decay_after_write:
                        S = (S + np.outer(bt * (vt - S @ kt), kt)) * a
                    else:
                        S = Sd + np.outer(u, kt)
                    if not read_before_write:
                        o[b, h, t] = S @ qt
                Sout[b, h] = S
        return o, Sout

    return forward


def _transposed_state_forward(q, k, v, g, beta, S0=None):
    """Mistake: keeps the state as d_k x d_v and reads o = S^T q from the wrong side."""
    o, S = oracle_forward(q, k, v, g, beta, S0)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if dk != dv:
        return o * np.nan, S
    # recompute reads with the transposed state at every prefix
    o2 = np.zeros_like(o)
    for t in range(T):
        _, St = oracle_forward(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1], g[:, :, :t + 1],
                               beta[:, :, :t + 1], S0)
        o2[:, :, t] = np.einsum("bhcv,bhc->bhv", St, q[:, :, t])
    return o2, S


MUTANTS = {
    "read_before_write": _python_recurrence(read_before_write=True),
    "prediction_from_undecayed_state": _python_recurrence(undecayed_prediction=True),
    "channel_decay_on_value_rows": _python_recurrence(kda_rows=True),
    "beta_dropped_from_prediction": _python_recurrence(drop_beta_in_prediction=True),
    "decay_after_write": _python_recurrence(decay_after_write=True),
    "transposed_read": _transposed_state_forward,
}


def _all_pins(fwd):
    res = {}
    for gate in GATES:
        for name, pin in (("p1", pin_p1_beta_zero), ("p2", pin_p2_identity_tokens), ("p4", pin_p4_beta_one),
                          ("p5", pin_p5_orthonormal_keys), ("p6", pin_p6_mix_identity),
                          ("dense", pin_dense_transition), ("p12", pin_p12_linearity), ("p13", pin_p13_split)):
            with np.errstate(all="ignore"):
                res[f"{name}_{gate}"] = pin(fwd, gate)
    with np.errstate(all="ignore"):
        res["p3"] = pin_p3_deltanet(fwd)
        res["p3_square"] = pin_p3_deltanet(fwd, dk=5, dv=5)
        res["p11"] = pin_p11_first_rows(fwd)
        res["alice_bob"] = pin_alice_bob(fwd)
    return res


def test_correct_python_recurrence_passes_pins():
    """The mutant harness itself, with no mistake planted, passes every pin."""
    res = _all_pins(_python_recurrence())
    assert all(v < 1e-10 for v in res.values()), res


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(mutant):
    res = _all_pins(MUTANTS[mutant])
    failed = [k for k, v in res.items() if not (v < 1e-8)]
    assert failed, f"mutant {mutant} passed every pin: {res}"
