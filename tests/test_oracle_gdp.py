"""Pins for the Gated Delta Product oracle (runs without a GPU).

``oracle.gdp_forward`` follows "Linear Attention, Visualized", section "Gated
Delta Product (GDP)": per real token, one decay and then n_h ordered
generalized-Householder substeps, the query read after the last one.  The checks
below do not reuse it:

* n_h = 1 is Gated DeltaNet: the token recurrence of ``oracle.recurrent_forward``,
  a separately written C routine (column convention, rank-one updates, no
  explicit transition matrix);
* the page's claim that GDP is GDN over the virtual sequence of section "GDP as
  GDN over a virtual sequence" (every n_h, non-unit keys, beta up to 2);
* beta = 0: pure decay, closed form;
* reflections: unit keys, beta = 2, no decay, zero values -- each substep is an
  orthogonal reflection, so the state's Frobenius norm never changes;
* a two-substep example solved by hand (non-orthogonal keys, so the substep
  order, the place of the decay and the read position all change the numbers);
* the page's n_h = 3 table of virtual steps (``tests/golden/gdp_virtual_table.json``)
  for the mapping ``oracle.gdp_as_virtual_gdn``.

``test_gdp_planted_mistakes_fail_a_pin`` runs the same pins against a plain
Python GDP recurrence with one plausible mistake planted at a time.
"""
import json
import os

import numpy as np
import pytest

import oracle

TOL = 1e-12
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return None if x is None else np.asarray(x, dtype=np.float32).astype(np.float64)


def gdp_inputs(seed, B=1, H=2, T=6, nh=3, dk=5, dv=3, unit_k=False, beta_range=(0.0, 2.0),
               g_range=(-0.7, -0.01), s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, nh, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, nh, dv))
    beta = r.uniform(*beta_range, size=(B, H, T, nh))
    g = r.uniform(*g_range, size=(B, H, T))
    S0 = r.standard_normal((B, H, dv, dk)) * 0.5 if s0 else None
    return dict(q=f32(q), k=f32(k), v=f32(v), g=f32(g), beta=f32(beta), S0=f32(S0))


def scale(*xs):
    return max(1.0, *[float(np.max(np.abs(x))) for x in xs if x is not None])


# ----------------------------------------------------------------------------- pins
def pin_nh1_is_gdn(forward):
    """n_h = 1: one substep per token is exactly the Gated DeltaNet update."""
    x = gdp_inputs(1, T=9, nh=1, dk=6, dv=4)
    o, S = forward(**x)
    o2, S2 = oracle.recurrent_forward(x["q"], x["k"][:, :, :, 0], x["v"][:, :, :, 0], x["g"],
                                      x["beta"][:, :, :, 0], x["S0"])
    return max(np.max(np.abs(o - o2)), np.max(np.abs(S - S2))) / scale(o2, S2)


def pin_virtual_sequence(forward, nh=3):
    """GDP on T tokens equals GDN on the T n_h virtual steps, keeping every n_h-th output."""
    x = gdp_inputs(2 + nh, T=7, nh=nh, dk=5, dv=3)
    o, S = forward(**x)
    qt, kt, vt, gt, bt, keep = oracle.gdp_as_virtual_gdn(x["q"], x["k"], x["v"], x["g"], x["beta"])
    o2, S2 = oracle.recurrent_forward(qt, kt, vt, gt, bt, x["S0"])
    return max(np.max(np.abs(o - o2[:, :, keep])), np.max(np.abs(S - S2))) / scale(o2, S2)


def pin_beta_zero(forward):
    """beta = 0 on every substep: S_t = (prod_{s<=t} a_s) S0 and o_t = S_t q_t."""
    x = gdp_inputs(3, T=8, nh=2, beta_range=(0.0, 0.0))
    o, S = forward(**x)
    cum = np.exp(np.cumsum(x["g"], axis=-1))                           # [B,H,T]
    o_ref = cum[..., None] * np.einsum("bhvc,bhtc->bhtv", x["S0"], x["q"])
    S_ref = cum[..., -1][..., None, None] * x["S0"]
    return max(np.max(np.abs(o - o_ref)), np.max(np.abs(S - S_ref))) / scale(o_ref, S_ref)


def pin_reflections(forward):
    """Unit keys, beta = 2, a = 1, v = 0: every substep is the reflection I - 2 k^T k,
    so ||S_t||_F = ||S_0||_F after each token (checked on every prefix)."""
    x = gdp_inputs(4, T=5, nh=3, dk=6, dv=4, beta_range=(2.0, 2.0), g_range=(0.0, 0.0))
    x["v"] = np.zeros_like(x["v"])
    # keys of exactly unit norm in binary: four entries of +-1/2 at random places
    r = np.random.default_rng(44)
    k = np.zeros_like(x["k"])
    for row in k.reshape(-1, k.shape[-1]):
        row[r.choice(k.shape[-1], size=4, replace=False)] = r.choice([-0.5, 0.5], size=4)
    x["k"] = k
    n0 = np.linalg.norm(x["S0"], axis=(-2, -1))
    errs = []
    for t in range(1, x["q"].shape[2] + 1):
        xt = {key: (val if key == "S0" else val[:, :, :t]) for key, val in x.items()}
        _, S = forward(**xt)
        errs.append(np.max(np.abs(np.linalg.norm(S, axis=(-2, -1)) - n0)))
    # and the reflections are not the identity: the state does move
    moved = np.max(np.abs(S - x["S0"]))
    return max(errs) / scale(n0) + (0.0 if moved > 0.1 else 1.0)


def pin_hand_example(forward):
    """d_k = 2, d_v = 1, n_h = 2, one token, solved by hand in the page's row notation,
    with the decay a = exp(g) kept as a symbol (g = log 1/2 rounded to float32).

    P0 = S0^T = (4, 6)^T; substep 1: k = e1, v = 1, beta = 1; substep 2: k = (1, 1)
    (not unit), v = 2, beta = 1/2; q = (1, 3).
      decay:      P = (4a, 6a)^T
      substep 1:  (I - e1 e1^T) P + e1 * 1                        = (1, 6a)^T
      substep 2:  (I - k k^T / 2) P + k * 2 / 2 = (1/2 - 3a, 3a - 1/2)^T + (1, 1)^T
                                                                  = (3/2 - 3a, 1/2 + 3a)^T
      o = q P = 3 + 6a.
    Every value here is exact in binary, so the pin is tight.
    """
    g = np.float32(np.log(0.5))
    a = float(np.exp(np.float64(g)))
    x = dict(q=np.array([1.0, 3.0]).reshape(1, 1, 1, 2),
             k=np.array([[1.0, 0.0], [1.0, 1.0]]).reshape(1, 1, 1, 2, 2),
             v=np.array([1.0, 2.0]).reshape(1, 1, 1, 2, 1),
             g=np.full((1, 1, 1), np.float64(g)),
             beta=np.array([1.0, 0.5]).reshape(1, 1, 1, 2),
             S0=np.array([4.0, 6.0]).reshape(1, 1, 1, 2))
    o, S = forward(**x)
    return max(abs(o[0, 0, 0, 0] - (3 + 6 * a)), np.max(np.abs(S[0, 0, 0] - [1.5 - 3 * a, 0.5 + 3 * a])))


def _all_pins(forward):
    with np.errstate(all="ignore"):
        return {"nh1": pin_nh1_is_gdn(forward), "virtual2": pin_virtual_sequence(forward, 2),
                "virtual3": pin_virtual_sequence(forward, 3), "virtual4": pin_virtual_sequence(forward, 4),
                "beta0": pin_beta_zero(forward), "reflect": pin_reflections(forward),
                "hand": pin_hand_example(forward)}


# ----------------------------------------------------------------------------- oracle tests
def test_gdp_oracle_passes_every_pin():
    res = _all_pins(oracle.gdp_forward)
    assert all(val < TOL for val in res.values()), res


@pytest.mark.parametrize("nh", [1, 2, 3, 5])
def test_gdp_virtual_sequence_with_unit_keys(nh):
    """The virtual-sequence identity on unit keys and the workloads' beta range, d_k != d_v."""
    x = gdp_inputs(40 + nh, B=2, H=1, T=11, nh=nh, dk=7, dv=4, unit_k=True, beta_range=(0.0, 1.0))
    o, S = oracle.gdp_forward(**x)
    qt, kt, vt, gt, bt, keep = oracle.gdp_as_virtual_gdn(x["q"], x["k"], x["v"], x["g"], x["beta"])
    o2, S2 = oracle.recurrent_forward(qt, kt, vt, gt, bt, x["S0"])
    assert np.max(np.abs(o - o2[:, :, keep])) < TOL * scale(o2)
    assert np.max(np.abs(S - S2)) < TOL * scale(S2)


def test_gdp_empty_sequence_returns_initial_state():
    x = gdp_inputs(7, T=0, nh=2)
    o, S = oracle.gdp_forward(**x)
    assert o.shape == (1, 2, 0, 3)
    assert np.array_equal(S, x["S0"])


def test_gdp_virtual_table_matches_page():
    """The mapping against the page's n_h = 3, two-token table."""
    with open(os.path.join(GOLDEN, "gdp_virtual_table.json")) as fh:
        tab = json.load(fh)
    nh, T, dk, dv = tab["n_h"], tab["T"], 4, 2
    r = np.random.default_rng(11)
    q = f32(r.standard_normal((1, 1, T, dk)))
    k = f32(r.standard_normal((1, 1, T, nh, dk)))
    v = f32(r.standard_normal((1, 1, T, nh, dv)))
    beta = f32(r.uniform(0.1, 0.9, size=(1, 1, T, nh)))
    g = f32(np.log([[[0.25, 0.75]]]))
    qt, kt, vt, gt, bt, keep = oracle.gdp_as_virtual_gdn(q, k, v, g, beta)
    assert kt.shape[2] == len(tab["virtual_steps"]) == T * nh
    for row in tab["virtual_steps"]:
        m, t, j = row["m"] - 1, row["t"] - 1, row["j"] - 1
        assert m == nh * t + j
        assert np.array_equal(kt[0, 0, m], k[0, 0, t, j])
        assert np.array_equal(vt[0, 0, m], v[0, 0, t, j])
        assert bt[0, 0, m] == beta[0, 0, t, j]
        a = float(np.exp(gt[0, 0, m]))
        want_a = float(np.exp(g[0, 0, t])) if row["decay"].startswith("a_") else 1.0
        assert abs(a - want_a) < 1e-7
        if row["query"] == "0":
            assert not np.any(qt[0, 0, m])
        else:
            assert row["query"] == f"q_{t + 1}" and np.array_equal(qt[0, 0, m], q[0, 0, t])
        assert (m in set(keep.tolist())) == (row["kept_output"] is not None)
    assert list(keep) == [row["m"] - 1 for row in tab["virtual_steps"] if row["kept_output"]]


# ----------------------------------------------------------------------------- planted mistakes
def _python_gdp(decay_each_substep=False, decay_after=False, reversed_substeps=False, read_early=False,
                plus_householder=False, value_unscaled=False):
    """A plain Python GDP recurrence (row notation, P = S^T) with switchable mistakes."""
    def forward(q, k, v, g, beta, S0=None):
        B, H, T, dk = q.shape
        nh, dv = k.shape[3], v.shape[-1]
        o = np.zeros((B, H, T, dv))
        S = np.zeros((B, H, dv, dk))
        for b in range(B):
            for h in range(H):
                P = np.zeros((dk, dv)) if S0 is None else S0[b, h].T.copy()
                for t in range(T):
                    a = np.exp(g[b, h, t])
                    if not (decay_each_substep or decay_after):
                        P = a * P
                    order = range(nh - 1, -1, -1) if reversed_substeps else range(nh)
                    for n, j in enumerate(order):
                        kk = k[b, h, t, j][:, None]
                        vv = v[b, h, t, j][None, :]
                        be = beta[b, h, t, j]
                        if decay_each_substep:
                            P = a * P
                        if read_early and n == nh - 1:
                            o[b, h, t] = q[b, h, t] @ P
                        sign = 1.0 if plus_householder else -1.0
                        P = (np.eye(dk) + sign * be * kk @ kk.T) @ P + (1.0 if value_unscaled else be) * kk @ vv
                    if decay_after:
                        P = a * P
                    if not read_early:
                        o[b, h, t] = q[b, h, t] @ P
                S[b, h] = P.T
        return o, S
    return forward


MUTANTS = {
    "decay_each_substep": _python_gdp(decay_each_substep=True),
    "decay_after_substeps": _python_gdp(decay_after=True),
    "reversed_substeps": _python_gdp(reversed_substeps=True),
    "read_before_last_substep": _python_gdp(read_early=True),
    "householder_sign": _python_gdp(plus_householder=True),
    "value_without_beta": _python_gdp(value_unscaled=True),
}


def test_gdp_python_recurrence_passes_pins():
    res = _all_pins(_python_gdp())
    assert all(val < 1e-10 for val in res.values()), res


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_gdp_planted_mistakes_fail_a_pin(mutant):
    res = _all_pins(MUTANTS[mutant])
    failed = [key for key, val in res.items() if not (val < 1e-8)]
    assert failed, f"mutant {mutant} passed every pin: {res}"
