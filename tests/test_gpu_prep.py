"""GPU parity of the chunked forward with fused input preparation (gdr_chunk_fwd_fused_prep).

The oracle side prepares the inputs with ``oracle.prepare_inputs`` (unit-norm q and k,
beta = sigmoid, Mamba-2 gate) in fp64 and runs the fp64 token recurrence on them; the GPU
side gets the raw projections.  Bars: tests/parity.py.
"""
import dataclasses

import numpy as np
import pytest

import gdr_synth
import oracle
from parity import TOL_BF16, err_bf16_out, err_literal, report

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gated_delta_rule_15_amd as gdr  # noqa: E402

DEV = torch.device("cuda:0")


def dev(a, bf16=False):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def variant(**kw):
    return dataclasses.replace(gdr_synth.WORKLOADS[2], **kw)


def run(r, S0=None, **kw):
    o, S = gdr.chunk_fwd_fused_prep(dev(r["q_raw"], True), dev(r["k_raw"], True), dev(r["v"], True), dev(r["dt"]),
                                    dev(r["A_log"]), dev(r["dt_bias"]), dev(r["beta_logit"]), dev(S0), **kw)
    torch.cuda.synchronize()
    return o, S


def ref(r, S0=None):
    q, k, g, beta = oracle.prepare_inputs(r["q_raw"], r["k_raw"], r["dt"], r["A_log"], r["dt_bias"], r["beta_logit"])
    return oracle.recurrent_forward(q, k, r["v"], g, beta, S0)


def check(name, o, S, o_ref, S_ref):
    eo, es, msg = report(name, host(o), o_ref, None if S is None else host(S), S_ref, True)
    print(msg)
    assert eo <= TOL_BF16 and es <= TOL_BF16, msg




def state(seed, B, H, dv, dk, std=0.05):
    return (np.random.default_rng(seed).standard_normal((B, H, dv, dk)) * std).astype(np.float32)


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 32), (64, 64), (64, 96)])
@pytest.mark.parametrize("with_s0", [False, True])
def test_prep_small(T, dk, dv, with_s0):
    r = gdr_synth.make_raw_inputs(variant(d_k=dk, d_v=dv), B=2, H=3, T=T, head_params="varied")
    S0 = state(T, 2, 3, dv, dk) if with_s0 else None
    o, S = run(r, S0)
    o_ref, S_ref = ref(r, S0)
    check(f"fused prep T={T} dk={dk} dv={dv} s0={with_s0}", o, S, o_ref, S_ref)


def test_prep_matches_unfused_path():
    """Preparing the inputs separately (fp32 on the host, q and k rounded to bf16) and calling
    gdr_chunk_fwd gives the same result within the output's bf16 rounding."""
    r = gdr_synth.make_raw_inputs(variant(), B=1, H=4, T=300, head_params="varied")
    o, S = run(r)
    q, k, g, beta = oracle.prepare_inputs(r["q_raw"], r["k_raw"], r["dt"], r["A_log"], r["dt_bias"], r["beta_logit"])
    o2, S2 = gdr.chunk_fwd(dev(q.astype(np.float32), True), dev(k.astype(np.float32), True), dev(r["v"], True),
                           dev(g.astype(np.float32)), dev(beta.astype(np.float32)))
    torch.cuda.synchronize()
    o_ref, S_ref = ref(r)
    check("fused prep", o, S, o_ref, S_ref)
    check("prepared then chunk_fwd", o2, S2, o_ref, S_ref)
    assert err_bf16_out(host(o), host(o2)) <= TOL_BF16


def test_prep_zero_and_large_raw_vectors():
    """Zero raw q / k rows give zero vectors (as the oracle's eps rule); raw magnitudes of
    10^3 normalise exactly like unit-scale ones."""
    r = gdr_synth.make_raw_inputs(variant(), B=1, H=2, T=130, head_params="varied")
    r["k_raw"][0, 0, 5] = 0.0
    r["q_raw"][0, 1, 70] = 0.0
    r["k_raw"][0, 1, 100:110] *= 1000.0
    r["q_raw"][0, 0, 20:30] *= 1e-3
    r["k_raw"] = gdr_synth.round_to_bf16(r["k_raw"])
    r["q_raw"] = gdr_synth.round_to_bf16(r["q_raw"])
    o, S = run(r)
    o_ref, S_ref = ref(r)
    check(f"fused prep, zero and scaled rows", o, S, o_ref, S_ref)


def test_prep_extreme_gate_parameters():
    """Raw gate inputs far outside the configs': dt of +-40 (softplus of 40, a decay of e^-40
    per token, and softplus of -40, no decay at all), saturated beta logits (+-40, so beta is
    1 or about 4e-18) and a head with lambda = e^3; the preparation's softplus and logistic
    map must stay finite and match the oracle's."""
    r = gdr_synth.make_raw_inputs(variant(), B=1, H=2, T=200, head_params="varied")
    r["dt"][0, 0, 10:40] = 40.0
    r["dt"][0, 1, 50:120] = -40.0
    r["beta_logit"][0, 0, 60:90] = 40.0
    r["beta_logit"][0, 1, 130:160] = -40.0
    r["A_log"][1] = 3.0
    o, S = run(r)
    o_ref, S_ref = ref(r)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check("fused prep, extreme gate parameters", o, S, o_ref, S_ref)


def test_prep_full_size_sampled():
    """B=4, H=16, T=4096, d=128 from raw projections; 4 of the 64 sequences checked."""
    w = gdr_synth.WORKLOADS[2]
    r = gdr_synth.make_raw_inputs(w, head_params="varied")
    o, S = run(r)
    pick = np.array([3, 22, 41, 60])
    bi, hi = pick // w.H, pick % w.H
    sub = {kk: r[kk][bi, hi][None] for kk in ("q_raw", "k_raw", "v", "dt", "beta_logit")}
    q, k, g, beta = oracle.prepare_inputs(sub["q_raw"], sub["k_raw"], sub["dt"], r["A_log"][hi], r["dt_bias"][hi],
                                          sub["beta_logit"])
    o_ref, S_ref = oracle.recurrent_forward(q, k, sub["v"], g, beta)
    o_s = o[torch.from_numpy(bi), torch.from_numpy(hi)][None]
    S_s = S[torch.from_numpy(bi), torch.from_numpy(hi)][None]
    check(f"fused prep full size, (4 sampled heads)", o_s, S_s, o_ref, S_ref)


def test_prep_carried_state_split():
    r = gdr_synth.make_raw_inputs(variant(), B=1, H=2, T=260, head_params="varied")
    S0 = state(3, 1, 2, 128, 128, std=0.02)
    o_ref, S_ref = ref(r, S0)
    t0 = 100
    per_tok = ("q_raw", "k_raw", "v", "dt", "beta_logit")
    a = {kk: (r[kk][:, :, :t0] if kk in per_tok else r[kk]) for kk in r}
    b = {kk: (r[kk][:, :, t0:] if kk in per_tok else r[kk]) for kk in r}
    oa, Sa = run(a, S0)
    ob, Sb = gdr.chunk_fwd_fused_prep(dev(b["q_raw"], True), dev(b["k_raw"], True), dev(b["v"], True), dev(b["dt"]),
                                      dev(b["A_log"]), dev(b["dt_bias"]), dev(b["beta_logit"]), Sa)
    torch.cuda.synchronize()
    check(f"fused prep split at {t0}", torch.cat([oa, ob], dim=2), Sb, o_ref, S_ref)


def test_prep_empty_sequence_copies_state():
    r = gdr_synth.make_raw_inputs(variant(), B=1, H=2, T=0)
    S0 = state(4, 1, 2, 128, 128)
    o, S = run(r, S0)
    assert o.numel() == 0 and torch.equal(S.cpu(), torch.from_numpy(S0))




def test_prep_full_grid_small_T():
    """B=4, H=16: the grid the state pass serves with two consumer waves per workgroup."""
    r = gdr_synth.make_raw_inputs(variant(), B=4, H=16, T=150, head_params="varied")
    o, S = run(r)
    o_ref, S_ref = ref(r)
    check("fused prep full grid, T=150", o, S, o_ref, S_ref)
