"""GPU parity of the Gated Delta Product forward (gdr_gdp_chunk_fwd) against the fp64 oracle.

Small cases compare every element with the token-wise GDP oracle (``oracle.gdp_forward``),
with n_h values that make real tokens straddle 64-step chunk boundaries and ragged tails.
The full-size workload (B=4, H=16, T=2048, n_h=2, d=128) runs in the launch configuration
the bench times; sampled sequences are checked against GDN over the virtual sequence
(``oracle.gdp_as_virtual_gdn`` + ``oracle.recurrent_forward``, pinned equal to the
token-wise oracle on the CPU).  Bars: tests/parity.py.
"""
import dataclasses

import numpy as np
import pytest

import gdr_synth
import oracle
from parity import TOL_BF16, report

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
    return dataclasses.replace(gdr_synth.WORKLOADS[6], **kw)


def run_gdp(x, S0=None, **kw):
    o, S = gdr.gdp_chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]),
                             dev(x["beta"]), dev(S0), **kw)
    torch.cuda.synchronize()
    return o, S


def check(name, o, S, o_ref, S_ref):
    eo, es, msg = report(name, host(o), o_ref, None if S is None else host(S), S_ref, True)
    print(msg)
    assert eo <= TOL_BF16 and es <= TOL_BF16, msg




def state(seed, B, H, dv, dk, std=0.05):
    return (np.random.default_rng(seed).standard_normal((B, H, dv, dk)) * std).astype(np.float32)


@pytest.mark.parametrize("T", [1, 22, 43, 100])
@pytest.mark.parametrize("nh", [2, 3, 4])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 96)])
@pytest.mark.parametrize("with_s0", [False, True])
def test_gdp_small(T, nh, dk, dv, with_s0):
    w = variant(nh=nh, d_k=dk, d_v=dv)
    x = gdr_synth.make_inputs(w, B=2, H=2, T=T)
    S0 = state(T + nh, 2, 2, dv, dk) if with_s0 else None
    o, S = run_gdp(x, S0)
    o_ref, S_ref = oracle.gdp_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"gdp T={T} nh={nh} dk={dk} dv={dv} s0={with_s0}", o, S, o_ref, S_ref)


@pytest.mark.parametrize("nh,T", [(5, 30), (16, 9), (7, 64)])
def test_gdp_many_substeps(nh, T):
    w = variant(nh=nh)
    x = gdr_synth.make_inputs(w, B=1, H=2, T=T)
    S0 = state(nh, 1, 2, 128, 128)
    o, S = run_gdp(x, S0)
    o_ref, S_ref = oracle.gdp_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"gdp nh={nh} T={T}", o, S, o_ref, S_ref)


@pytest.mark.parametrize("kind", ["reflections", "identity", "mixed"])
def test_gdp_special_substeps(kind):
    """beta = 2 with unit keys makes every substep a Householder reflection I - 2 k k^T (a swap
    of two coordinates for k = (e_a - e_b)/sqrt(2), "A Swap Is a Reflection"); beta = 0 makes
    it the identity (only the decay acts); mixed takes 0, 2 and the drawn values in turn."""
    w = variant(nh=3)
    x = gdr_synth.make_inputs(w, B=1, H=2, T=70)
    if kind == "reflections":
        x["beta"][:] = 2.0
    elif kind == "identity":
        x["beta"][:] = 0.0
    else:
        x["beta"][..., 0] = 0.0
        x["beta"][..., 1] = 2.0
    S0 = state(11, 1, 2, 128, 128, std=0.2)
    o, S = run_gdp(x, S0)
    o_ref, S_ref = oracle.gdp_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"gdp {kind} substeps", o, S, o_ref, S_ref)


def test_gdp_equals_chunk_fwd_on_the_virtual_sequence():
    """The GDP kernels read q, g and write o through the substep mapping; fed the expanded
    virtual sequence, the chunked forward on the same path (the same kernel bodies) must give
    the same bits."""
    w = variant(nh=3)
    x = gdr_synth.make_inputs(w, B=2, H=3, T=150)
    S0 = state(3, 2, 3, 128, 128)
    o, S = run_gdp(x, S0)
    qt, kt, vt, gt, bt, keep = oracle.gdp_as_virtual_gdn(x["q"], x["k"], x["v"], x["g"], x["beta"])
    ov, Sv = gdr.chunk_fwd(dev(qt, True), dev(kt, True), dev(vt, True), dev(gt), dev(bt), dev(S0))
    torch.cuda.synchronize()
    assert torch.equal(o, ov[:, :, torch.from_numpy(keep).to(DEV)])
    assert torch.equal(S, Sv)


def test_gdp_one_substep_is_chunk_fwd():
    w = variant(nh=1)
    x = gdr_synth.make_inputs(w, B=1, H=4, T=200)
    o, S = gdr.gdp_chunk_fwd(dev(x["q"], True), dev(x["k"][:, :, :, None], True), dev(x["v"][:, :, :, None], True),
                             dev(x["g"]), dev(x["beta"][:, :, :, None]))
    o2, S2 = gdr.chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]), dev(x["beta"]))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2)


def test_gdp_full_size_sampled():
    """B=4, H=16, T=2048, n_h=2, d=128 bf16 (4096 substeps per sequence); 6 of 64 sequences."""
    w = gdr_synth.WORKLOADS[6]
    x = gdr_synth.make_inputs(w)
    o, S = run_gdp(x)
    rng = np.random.default_rng(6)
    pick = np.sort(rng.choice(w.B * w.H, size=6, replace=False))
    bi, hi = pick // w.H, pick % w.H
    sub = {kk: x[kk][bi, hi][None] for kk in ("q", "k", "v", "g", "beta")}
    qt, kt, vt, gt, bt, keep = oracle.gdp_as_virtual_gdn(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"])
    o_ref, S_ref = oracle.recurrent_forward(qt, kt, vt, gt, bt)
    o_s = o[torch.from_numpy(bi), torch.from_numpy(hi)][None]
    S_s = S[torch.from_numpy(bi), torch.from_numpy(hi)][None]
    check(f"gdp full size, (6 sampled heads)", o_s, S_s, o_ref[:, :, keep], S_ref)


def test_gdp_carried_state_split():
    """gdp(x[:t0]) then gdp(x[t0:], S) matches the oracle on x."""
    w = variant(nh=3)
    x = gdr_synth.make_inputs(w, B=1, H=2, T=90)
    S0 = state(9, 1, 2, 128, 128)
    o_ref, S_ref = oracle.gdp_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    for t0 in (20, 43):
        a = {kk: vv[:, :, :t0] for kk, vv in x.items() if vv is not None}
        b = {kk: vv[:, :, t0:] for kk, vv in x.items() if vv is not None}
        oa, Sa = run_gdp(a, S0)
        ob, Sb = gdr.gdp_chunk_fwd(dev(b["q"], True), dev(b["k"], True), dev(b["v"], True), dev(b["g"]),
                                   dev(b["beta"]), Sa)
        torch.cuda.synchronize()
        check(f"gdp split at {t0}", torch.cat([oa, ob], dim=2), Sb, o_ref, S_ref)


def test_gdp_empty_sequence_copies_state():
    x = gdr_synth.make_inputs(variant(nh=2), B=1, H=2, T=0)
    S0 = state(4, 1, 2, 128, 128)
    o, S = run_gdp(x, S0)
    assert o.numel() == 0 and torch.equal(S.cpu(), torch.from_numpy(S0))


def test_gdp_deterministic():
    x = gdr_synth.make_inputs(variant(nh=3), B=1, H=4, T=120)
    o1, S1 = run_gdp(x)
    o2, S2 = run_gdp(x)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_gdp_explicit_workspace_reused():
    """A caller-owned workspace reused across calls of different sizes."""
    need = gdr.gdp_chunk_fwd_workspace_size(1, 2, 120, 3, 128, 128)
    wsb = torch.empty(need, dtype=torch.uint8, device=DEV)
    for T, nh in ((120, 3), (43, 2), (9, 16)):
        x = gdr_synth.make_inputs(variant(nh=nh), B=1, H=2, T=T)
        o, S = run_gdp(x, workspace=wsb)
        o_ref, S_ref = oracle.gdp_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
        check(f"gdp reused workspace T={T} nh={nh}", o, S, o_ref, S_ref)
