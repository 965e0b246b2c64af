"""GPU parity at the edges of the method's inputs, through the C ABI, against the fp64 oracle.

The configs' distributions (beta = sigmoid(N(0,1)), small decays, unit keys, v ~ N(0,1)) leave
out cases the pages single out:
  * beta = 0 (no write: pure decay), beta = 1 with unit keys (exact write, S_t k_t = v_t),
    beta = 2 (a Householder reflection: "A Swap Is a Reflection"), an erase gate up to 2
    ("Gated DeltaNet-2 ...", section 2);
  * alpha = 1 (g = 0: plain DeltaNet) and g = 0 with beta = 0 (identity tokens);
  * keys that are not unit norm (the kernels do not normalise) and runs of near-parallel keys
    with beta close to 1, where the triangular system of the UT transform is least benign
    ("Gated DeltaNet: Householder Transitions...", "The part that could have killed it");
  * v and the initial state scaled by 2^-14 and 2^12: the recurrence is affine in S with a
    write linear in v (the video delta-rule post, Preliminaries), so (o, S_T) must scale
    exactly (P12 in the oracle pins) whatever the fp16 operand range;
  * per-channel log-decays far steeper than the configs' (down to -100 per token, and a
    single near-reset token), which "Linear Attention, Visualized", section "Kimi Delta
    Attention (KDA)", allows for any a_t in (0, 1];
  * a NaN in one token, which must stay inside its own sequence;
  * a small positive log-decay (a_t slightly above 1) over a short sequence.
Every case compares element by element with the oracle at the bars of tests/parity.py.
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


def bf(x):
    return gdr_synth.round_to_bf16(np.asarray(x, dtype=np.float32))


def variant(wid, **kw):
    return dataclasses.replace(gdr_synth.WORKLOADS[wid], **kw)


def run(x, S0=None):
    o, S = gdr.chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]), dev(x["beta"]),
                         dev(S0))
    torch.cuda.synchronize()
    return o, S


def check(name, o, S, o_ref, S_ref):
    eo, es, msg = report(name, host(o), o_ref, host(S), S_ref, True)
    print(msg)
    assert eo <= TOL_BF16 and es <= TOL_BF16, msg


def err_one_ulp(x, ref):
    """max_i (|x_i - ref_i| - 2^-7 max(|x_i|, |ref_i|))_+ / RMS(ref): two bf16 results charged only
    beyond one bf16 unit in the last place (two roundings of nearly equal values may differ by
    one)."""
    d = np.abs(x - ref) - 2.0 ** -7 * np.maximum(np.abs(x), np.abs(ref))
    return float(np.max(np.maximum(d, 0.0))) / max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)


def s0(seed, B, H, dv, dk, std=0.05):
    return (np.random.default_rng(seed).standard_normal((B, H, dv, dk)) * std).astype(np.float32)


# ----------------------------------------------------------------------------- gate values
@pytest.mark.parametrize("wid", [2, 3])
@pytest.mark.parametrize("beta", [0.0, 1.0, 2.0])
def test_constant_beta(wid, beta):
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=1, H=2, T=200)
    x["beta"][:] = beta
    S0 = s0(1, 1, 2, 128, 128)
    o, S = run(x, S0)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"workload {wid} gate, beta = {beta}", o, S, o_ref, S_ref)
    if beta == 1.0:
        # exact write (P4): the last token's key reads its value back from the final state
        k, v = x["k"][0, :, -1].astype(np.float64), x["v"][0, :, -1].astype(np.float64)
        got = np.einsum("hvc,hc->hv", host(S)[0], k)
        assert np.max(np.abs(got - v)) <= 2e-2 * np.sqrt(np.mean(v ** 2)), np.max(np.abs(got - v))


@pytest.mark.parametrize("wid", [2, 3])
def test_no_decay_is_deltanet(wid):
    """alpha = 1 (g = 0): plain DeltaNet, the page's P3 case."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=1, H=2, T=300)
    x["g"][:] = 0.0
    o, S = run(x)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    check(f"workload {wid} gate, g = 0", o, S, o_ref, S_ref)


@pytest.mark.parametrize("wid", [2, 3])
def test_identity_tokens(wid):
    """g = 0 and beta = 0 on every token: the state passes through, o_t = S0 q_t."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=1, H=2, T=130)
    x["g"][:] = 0.0
    x["beta"][:] = 0.0
    S0 = s0(2, 1, 2, 128, 128)
    o, S = run(x, S0)
    assert torch.equal(S.cpu(), torch.from_numpy(S0))
    o_ref = np.einsum("bhvc,bhtc->bhtv", S0.astype(np.float64), x["q"].astype(np.float64))
    assert err_bf16_out(host(o), o_ref) <= TOL_BF16


# ----------------------------------------------------------------------------- keys
def test_non_unit_keys():
    """Keys of norm 0.5 .. 1.4 (the kernels do not normalise) with beta <= 0.9, so that
    beta ||k||^2 < 2 keeps every token's transition a contraction."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=1, H=2, T=260)
    r = np.random.default_rng(3).uniform(0.5, 1.4, size=x["k"].shape[:-1] + (1,))
    x["k"] = bf(x["k"] * r)
    x["beta"] = (0.9 * x["beta"]).astype(np.float32)
    S0 = s0(3, 1, 2, 128, 128)
    o, S = run(x, S0)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check("non-unit keys", o, S, o_ref, S_ref)


@pytest.mark.parametrize("wid", [2, 3])
@pytest.mark.parametrize("eps", [1e-2, 1e-3])
def test_near_parallel_keys(wid, eps):
    """Runs of 8 consecutive tokens whose unit keys differ by eps, with beta = 0.99: the
    Gram matrix of a run is nearly singular and N's off-diagonal entries approach -1."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=1, H=2, T=256)
    rng = np.random.default_rng(4)
    B, H, T, dk = x["k"].shape
    base = np.repeat(rng.standard_normal((B, H, T // 8, 1, dk)), 8, axis=3).reshape(B, H, T, dk)
    k = base + eps * rng.standard_normal((B, H, T, dk))
    x["k"] = bf(k / np.linalg.norm(k, axis=-1, keepdims=True))
    x["beta"][:] = 0.99
    o, S = run(x)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    check(f"workload {wid} gate, near-parallel keys eps={eps}", o, S, o_ref, S_ref)


# ----------------------------------------------------------------------------- scale of v and S0
SCALES = [2.0 ** -14, 2.0 ** 12]


@pytest.mark.parametrize("wid", [2, 3, 4])
@pytest.mark.parametrize("scale", SCALES)
def test_scale_of_values_and_state(wid, scale):
    """(o, S_T) is linear in (v, S0): scaling both by a power of two scales the result
    exactly.  Checked against the oracle on the scaled inputs, and against the GPU's own
    unscaled result (the kernels' fp16 operands then differ by a power of two, so the two
    results agree to fp32 rounding before o's bf16 rounding)."""
    w = gdr_synth.WORKLOADS[wid]
    x = gdr_synth.make_inputs(w, B=1, H=2, T=300)
    S0 = s0(5, 1, 2, 128, 128, std=0.3)
    o1, S1 = run(x, S0)
    xs = dict(x)
    xs["v"] = (x["v"] * np.float32(scale)).astype(np.float32)
    S0s = (S0 * np.float32(scale)).astype(np.float32)
    o2, S2 = run(xs, S0s)
    o_ref, S_ref = oracle.recurrent_forward(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], S0s)
    check(f"workload {wid} gate, v and S0 times {scale:g}", o2, S2, o_ref, S_ref)
    assert err_one_ulp(host(o2) / scale, host(o1)) <= 1e-3
    assert err_literal(host(S2) / scale, host(S1)) <= 1e-3


@pytest.mark.parametrize("scale", SCALES)
def test_scale_gdp_and_gdn2(scale):
    """The Gated Delta Product and Gated DeltaNet-2 passes share the state kernel's scaling."""
    x = gdr_synth.make_inputs(variant(6, nh=2), B=1, H=2, T=100)
    S0 = (s0(6, 1, 2, 128, 128, std=0.3) * np.float32(scale)).astype(np.float32)
    v = (x["v"] * np.float32(scale)).astype(np.float32)
    o, S = gdr.gdp_chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(v, True), dev(x["g"]), dev(x["beta"]),
                             dev(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdp_forward(x["q"], x["k"], v, x["g"], x["beta"], S0)
    check(f"gdp, v and S0 times {scale:g}", o, S, o_ref, S_ref)
    y = gdr_synth.make_inputs(gdr_synth.WORKLOADS[7], B=1, H=2, T=200)
    v = (y["v"] * np.float32(scale)).astype(np.float32)
    o, S = gdr.gdn2_chunk_fwd(dev(y["q"], True), dev(y["k"], True), dev(v, True), dev(y["g"]), dev(y["b"]),
                              dev(y["w"]), dev(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn2_forward(y["q"], y["k"], v, y["g"], y["b"], y["w"], S0)
    check(f"gdn2, v and S0 times {scale:g}", o, S, o_ref, S_ref)


@pytest.mark.parametrize("scale", SCALES)
def test_scale_fused_prep(scale):
    r = gdr_synth.make_raw_inputs(gdr_synth.WORKLOADS[2], B=1, H=2, T=200, head_params="varied")
    v = (r["v"] * np.float32(scale)).astype(np.float32)
    o, S = gdr.chunk_fwd_fused_prep(dev(r["q_raw"], True), dev(r["k_raw"], True), dev(v, True), dev(r["dt"]),
                                    dev(r["A_log"]), dev(r["dt_bias"]), dev(r["beta_logit"]))
    torch.cuda.synchronize()
    q, k, g, beta = oracle.prepare_inputs(r["q_raw"], r["k_raw"], r["dt"], r["A_log"], r["dt_bias"], r["beta_logit"])
    o_ref, S_ref = oracle.recurrent_forward(q, k, v, g, beta)
    check(f"fused preparation, v times {scale:g}", o, S, o_ref, S_ref)


def test_values_jump_in_scale_mid_sequence():
    """v grows by 2^10 from one chunk to the next and shrinks back later: the operand scale
    must follow the chunk's values, not only the state carried in."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=1, H=2, T=320)
    x["v"][:, :, 64:128] *= np.float32(2.0 ** 10)
    x["v"][:, :, 192:] *= np.float32(2.0 ** -8)
    o, S = run(x)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    check("v scale jumps between chunks", o, S, o_ref, S_ref)


# ----------------------------------------------------------------------------- steep per-channel decay
@pytest.mark.parametrize("mode", ["kda", "gdn2"])
def test_steep_channel_decay(mode):
    """A few channels decay by e^-10 .. e^-100 per token, the rest at the configs' rate:
    the diagonal Gram tiles take the exact path, whose factors never exceed 1."""
    wid = 3 if mode == "kda" else 7
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=1, H=2, T=200)
    rng = np.random.default_rng(8)
    steep = rng.uniform(-100.0, -10.0, size=x["g"][..., ::5].shape).astype(np.float32)
    x["g"][..., ::5] = steep
    S0 = s0(8, 1, 2, 128, 128)
    if mode == "kda":
        o, S = run(x, S0)
        o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    else:
        o, S = gdr.gdn2_chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]),
                                  dev(x["b"]), dev(x["w"]), dev(S0))
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.gdn2_forward(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], S0)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(f"{mode}: channels with log-decay in U(-100, -10)", o, S, o_ref, S_ref)


@pytest.mark.parametrize("mode", ["kda", "gdn2"])
@pytest.mark.parametrize("pos", [3, 40, 64])
def test_near_reset_token(mode, pos):
    """One token with log-decay -90 on every channel (a near reset), inside a block, at a
    block's first token and at a chunk start."""
    wid = 3 if mode == "kda" else 7
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=1, H=2, T=150)
    x["g"][:, :, pos, :] = -90.0
    S0 = s0(9, 1, 2, 128, 128)
    if mode == "kda":
        o, S = run(x, S0)
        o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    else:
        o, S = gdr.gdn2_chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]),
                                  dev(x["b"]), dev(x["w"]), dev(S0))
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.gdn2_forward(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], S0)
    check(f"{mode}: near reset at token {pos}", o, S, o_ref, S_ref)


def test_steep_scalar_decay():
    """The scalar gate at log-decays down to -100 per token (its factors are e^{G_i - G_j},
    i >= j, throughout)."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=1, H=2, T=200)
    x["g"][..., ::7] = -np.random.default_rng(10).uniform(10.0, 100.0, size=x["g"][..., ::7].shape)
    o, S = run(x, s0(10, 1, 2, 128, 128))
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], s0(10, 1, 2, 128, 128))
    check("scalar gate with near resets", o, S, o_ref, S_ref)


# ----------------------------------------------------------------------------- positive gate
@pytest.mark.parametrize("wid", [2, 3])
def test_small_positive_log_decay(wid):
    """a_t slightly above 1 (g ~ U(0, 0.02)) over 150 tokens: accepted and computed (the
    factors e^{G_i - G_j} then exceed 1 by at most e^1.3 inside a chunk)."""
    x = gdr_synth.make_inputs(variant(wid, g_dist=("uniform", 0.0, 0.02)), B=1, H=2, T=150)
    o, S = run(x)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    check(f"workload {wid} gate, g ~ U(0, 0.02)", o, S, o_ref, S_ref)


# ----------------------------------------------------------------------------- non-finite inputs
@pytest.mark.parametrize("wid", [2, 3])
@pytest.mark.parametrize("field", ["v", "k", "g"])
def test_nan_stays_in_its_sequence(wid, field):
    """A NaN in one token of sequence (0, 1) leaves the other sequences' results bit-equal to
    a clean run, and the call completes."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=2, H=3, T=150)
    o1, S1 = run(x)
    y = {kk: (None if vv is None else vv.copy()) for kk, vv in x.items()}
    if field == "g" and y["g"].ndim == 4:
        y["g"][0, 1, 70, 5] = np.nan
    elif field == "g":
        y["g"][0, 1, 70] = np.nan
    else:
        y[field][0, 1, 70, 5] = np.nan
    o2, S2 = run(y)
    keep = torch.ones(2, 3, dtype=torch.bool)
    keep[0, 1] = False
    assert torch.equal(o1[keep], o2[keep]) and torch.equal(S1[keep], S2[keep])
    assert not torch.isfinite(S2[0, 1]).all()  # the NaN did reach its own sequence's state
