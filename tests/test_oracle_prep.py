"""Pins for the input-preparation oracle (``oracle.prepare_inputs``), CPU only.

It maps raw projections to the inputs of the gated delta rule: unit-norm q and k, beta =
sigmoid(logit), and Mamba-2's decay gate g = log a = -exp(A_log) softplus(dt + dt_bias)
("Linear Attention, Visualized", "Optional: Constructing the decay gate").  Checked against
closed forms and against the synthetic generator, which draws the same raw numbers and
transforms them in float32 with its own code.
"""
import dataclasses

import numpy as np

import gdr_synth
import oracle


def raw(seed, B=2, H=3, T=5, dk=8):
    r = np.random.default_rng(seed)
    return dict(q_raw=r.standard_normal((B, H, T, dk)) * 3.0, k_raw=r.standard_normal((B, H, T, dk)) * 0.1,
                dt=r.standard_normal((B, H, T)) * 2.0, A_log=r.uniform(-3.0, 1.0, size=H),
                dt_bias=r.standard_normal(H), beta_logit=r.standard_normal((B, H, T)) * 3.0)


def test_unit_norm_and_direction():
    x = raw(1)
    q, k, _, _ = oracle.prepare_inputs(**x)
    for y, y_raw in ((q, x["q_raw"]), (k, x["k_raw"])):
        assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
        cos = np.sum(y * y_raw, axis=-1) / np.linalg.norm(y_raw, axis=-1)
        assert np.allclose(cos, 1.0, rtol=0, atol=1e-14)         # same direction, positive


def test_zero_vector_stays_zero():
    x = raw(2)
    x["k_raw"][0, 1, 2] = 0.0
    _, k, _, _ = oracle.prepare_inputs(**x)
    assert not np.any(k[0, 1, 2]) and np.all(np.isfinite(k))


def test_beta_closed_forms():
    x = raw(3, T=4)
    x["beta_logit"][..., 0] = 0.0
    x["beta_logit"][..., 1] = np.log(3.0)
    x["beta_logit"][..., 2] = -np.log(3.0)
    x["beta_logit"][..., 3] = 40.0
    _, _, _, beta = oracle.prepare_inputs(**x)
    assert np.allclose(beta[..., 0], 0.5, atol=1e-15)
    assert np.allclose(beta[..., 1], 0.75, atol=1e-15)
    assert np.allclose(beta[..., 2], 0.25, atol=1e-15)
    assert np.all(beta[..., 3] <= 1.0) and np.allclose(beta[..., 3], 1.0, atol=1e-15)


def test_gate_closed_forms():
    """lambda = e^{A_log}, Delta = softplus(dt + b): A_log = log 2, b = 0, dt = 0 gives
    Delta = log 2 and a = e^{-2 log 2} = 1/4; dt = log(e - 1) gives Delta = 1, a = e^{-2};
    a large dt gives Delta ~ dt; a very negative one gives a -> 1 (g -> 0-)."""
    H = 1
    x = dict(q_raw=np.ones((1, H, 4, 2)), k_raw=np.ones((1, H, 4, 2)), beta_logit=np.zeros((1, H, 4)),
             A_log=np.array([np.log(2.0)]), dt_bias=np.zeros(H),
             dt=np.array([[[0.0, np.log(np.e - 1.0), 50.0, -60.0]]]))
    _, _, g, _ = oracle.prepare_inputs(**x)
    a = np.exp(g[0, 0])
    assert abs(a[0] - 0.25) < 1e-15
    assert abs(g[0, 0, 1] + 2.0) < 1e-14
    assert abs(g[0, 0, 2] + 100.0) < 1e-12
    assert -1e-25 < g[0, 0, 3] < 0.0


def test_gate_per_head_parameters_and_bias():
    """dt_bias shifts dt, A_log scales per head: g[h] = -e^{A_log[h]} softplus(dt + b[h])."""
    x = raw(4, H=3)
    _, _, g, _ = oracle.prepare_inputs(**x)
    for h in range(3):
        z = x["dt"][:, h] + x["dt_bias"][h]
        ref = -np.exp(x["A_log"][h]) * np.log1p(np.exp(z))
        assert np.allclose(g[:, h], ref, rtol=1e-14, atol=0)
    assert np.all(g < 0.0)


def test_matches_the_synthetic_generator():
    """The generator's float32 transforms of the same raw draws (workload 2 with f32 I/O,
    so no bf16 rounding intervenes) agree with the fp64 oracle to float32 precision."""
    w = dataclasses.replace(gdr_synth.WORKLOADS[2], io_dtype="f32")
    x = gdr_synth.make_inputs(w, B=2, H=3, T=50)
    r = gdr_synth.make_raw_inputs(w, B=2, H=3, T=50)
    q, k, g, beta = oracle.prepare_inputs(r["q_raw"], r["k_raw"], r["dt"], r["A_log"], r["dt_bias"],
                                          r["beta_logit"])
    assert np.max(np.abs(q - x["q"])) < 1e-6 and np.max(np.abs(k - x["k"])) < 1e-6
    assert np.max(np.abs(g - x["g"]) / np.abs(x["g"])) < 1e-6
    assert np.max(np.abs(beta - x["beta"])) < 1e-6
    assert np.array_equal(r["v"], x["v"])
