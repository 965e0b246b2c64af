"""GPU parity of the frame-level implicit update (gdr_frame_fwd) against the fp64 oracle
(``oracle.frame.frame_forward``: per frame a Cholesky factorisation of I + G and two
triangular solves, written from the video delta-rule post).  Bars: tests/parity.py."""
import numpy as np
import pytest

import gdr_synth
from oracle.frame import frame_forward
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


def run(x, n, **kw):
    o, S = gdr.frame_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["gamma"]), dev(x["g"]), n,
                         dev(x["S0"]), **kw)
    torch.cuda.synchronize()
    return o, S


def check(name, o, S, o_ref, S_ref):
    eo, es, msg = report(name, host(o), o_ref, None if S is None else host(S), S_ref, True)
    print(msg)
    assert eo <= TOL_BF16 and es <= TOL_BF16, msg


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("n,T", [(16, 48), (48, 150), (64, 256), (160, 330)])
@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("with_s0", [False, True])
def test_frame_small(dk, dv, n, T, channel, with_s0):
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=T, frame_len=n, d_k=dk, d_v=dv, channel=channel,
                                    s0_std=0.05 if with_s0 else 0.0, salt=n)
    o, S = run(x, n)
    o_ref, S_ref = frame_forward(x["q"], x["k"], x["v"], x["gamma"], x["g"], n, x["S0"])
    check(f"frame dk={dk} dv={dv} n={n} T={T} channel={channel} s0={with_s0}", o, S, o_ref, S_ref)


@pytest.mark.parametrize("scale", [0.01, 1.0, 30.0])
def test_frame_writing_strength_scales(scale):
    """Weak writes (near accumulation), about equal old state and frame, and strong writes
    that wipe the history (I + G far from the identity)."""
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=256, frame_len=64, channel=True, s0_std=0.05)
    x["gamma"] = (x["gamma"] * np.float32(scale)).astype(np.float32)
    o, S = run(x, 64)
    o_ref, S_ref = frame_forward(x["q"], x["k"], x["v"], x["gamma"], x["g"], 64, x["S0"])
    check(f"frame gamma x{scale}", o, S, o_ref, S_ref)


def test_frame_zero_writes_pure_decay():
    """gamma = 0: G = C = 0 and W = I, so each frame only decays the state, S_t = S_{t-1} D_t.
    Against the oracle, and S_T against the closed form S0 diag(exp(sum of the frame gates)),
    ragged last frame included."""
    n, T = 64, 200
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=T, frame_len=n, channel=True, s0_std=0.3)
    x["gamma"] = np.zeros_like(x["gamma"])
    o, S = run(x, n)
    o_ref, S_ref = frame_forward(x["q"], x["k"], x["v"], x["gamma"], x["g"], n, x["S0"])
    check("frame gamma = 0", o, S, o_ref, S_ref)
    closed = x["S0"].astype(np.float64) * np.exp(x["g"].astype(np.float64).sum(axis=2))[:, :, None, :]
    assert err_literal(host(S), closed) <= 1e-4


def test_frame_steep_channel_decays():
    """Per-channel log gates in U(-30, -10): the old state all but vanishes at every frame, so
    S_t is about C_t (I + G_t)^{-1}; the products of tiny decays must not lose the fresh part."""
    n, T = 64, 320
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=T, frame_len=n, channel=True, s0_std=0.05, salt=3)
    r = np.random.default_rng(5)
    x["g"] = r.uniform(-30.0, -10.0, size=x["g"].shape).astype(np.float32)
    o, S = run(x, n)
    o_ref, S_ref = frame_forward(x["q"], x["k"], x["v"], x["gamma"], x["g"], n, x["S0"])
    check("frame steep per-channel decays", o, S, o_ref, S_ref)


def test_frame_single_ragged_frame():
    """One frame longer than the sequence (frame_len 160, T = 150): every query reads the
    state after all 150 writes, through a partly filled last token block."""
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=150, frame_len=160, channel=False, s0_std=0.05, salt=4)
    o, S = run(x, 160)
    o_ref, S_ref = frame_forward(x["q"], x["k"], x["v"], x["gamma"], x["g"], 160, x["S0"])
    check("frame single ragged frame", o, S, o_ref, S_ref)


def test_frame_permutation_invariance():
    """Tokens permuted inside their frames: outputs permuted alike, final state unchanged
    (up to the fp32 summation order of G and C)."""
    n, T = 64, 320
    x = gdr_synth.make_frame_inputs(B=1, H=3, T=T, frame_len=n, channel=True)
    o, S = run(x, n)
    r = np.random.default_rng(1)
    perm = np.concatenate([f * n + r.permutation(min(n, T - f * n)) for f in range((T + n - 1) // n)])
    xp = {kk: (vv[:, :, perm] if kk in ("q", "k", "v", "gamma") else vv) for kk, vv in x.items()}
    op, Sp = run(xp, n)
    assert err_bf16_out(host(op), host(o)[:, :, perm]) <= 1e-2
    assert err_literal(host(Sp), host(S)) <= 1e-3


def test_frame_full_size_sampled():
    """B=1, H=16, T=16384 as 16 frames of 1024 tokens, d=128, per-channel gate; 3 heads."""
    w = gdr_synth.FRAME_WORKLOAD
    x = gdr_synth.make_frame_inputs(B=w["B"], H=w["H"], T=w["T"], frame_len=w["frame_len"], d_k=w["d_k"],
                                    d_v=w["d_v"])
    o, S = run(x, w["frame_len"])
    hi = np.array([0, 7, 15])
    sub = {kk: (None if vv is None else vv[:, hi]) for kk, vv in x.items()}
    o_ref, S_ref = frame_forward(sub["q"], sub["k"], sub["v"], sub["gamma"], sub["g"], w["frame_len"])
    check("frame full size (3 heads)", o[:, torch.from_numpy(hi)], S[:, torch.from_numpy(hi)], o_ref, S_ref)


def test_frame_carried_state_split():
    n = 64
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=448, frame_len=n, channel=True, s0_std=0.02)
    o_ref, S_ref = frame_forward(x["q"], x["k"], x["v"], x["gamma"], x["g"], n, x["S0"])
    t0 = 192  # a frame boundary
    f0 = t0 // n
    a = {kk: (vv if kk == "S0" else (vv[:, :, :f0] if kk == "g" else vv[:, :, :t0])) for kk, vv in x.items()}
    b = {kk: (None if kk == "S0" else (vv[:, :, f0:] if kk == "g" else vv[:, :, t0:])) for kk, vv in x.items()}
    oa, Sa = run(a, n)
    ob, Sb = gdr.frame_fwd(dev(b["q"], True), dev(b["k"], True), dev(b["v"], True), dev(b["gamma"]), dev(b["g"]), n,
                           Sa)
    torch.cuda.synchronize()
    check("frame split", torch.cat([oa, ob], dim=2), Sb, o_ref, S_ref)


def test_frame_empty_sequence_copies_state():
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=0, frame_len=16, s0_std=0.05)
    o, S = run(x, 16)
    assert o.numel() == 0 and torch.equal(S.cpu(), torch.from_numpy(x["S0"]))


def test_frame_deterministic():
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=300, frame_len=48)
    o1, S1 = run(x, 48)
    o2, S2 = run(x, 48)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("vscale", [50.0, 2.0 ** 10, 2.0 ** -14])
def test_frame_repeated_keys_strong_writes(vscale):
    """A static scene (the video delta-rule post, "A Different Route"): every frame repeats four
    (key, value) pairs, with writing strengths x30.  C = V^T Gamma K then grows with the frame
    length (about 1024 x 3.75 x |v| here) while the state stays near the values; v and S0 are
    also scaled by 2^10 and 2^-14, which the result must follow exactly (linearity).  The
    largest sqrt(gamma) |v| stays below fp16's 65504, the documented limit of the Gram kernel's
    operands."""
    n, T = 1024, 3072
    x = gdr_synth.make_frame_inputs(B=1, H=2, T=T, frame_len=n, channel=True, s0_std=0.05, salt=7)
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((1, 2, 4, 128)).astype(np.float32)
    keys /= np.linalg.norm(keys, axis=-1, keepdims=True)
    vals = rng.standard_normal((1, 2, 4, 128)).astype(np.float32)
    pick = rng.integers(0, 4, size=T)
    x["k"] = gdr_synth.round_to_bf16(keys[:, :, pick] + 0.01 * rng.standard_normal((1, 2, T, 128)).astype(np.float32))
    x["v"] = gdr_synth.round_to_bf16((vals[:, :, pick] + 0.1 * rng.standard_normal((1, 2, T, 128))).astype(np.float32)
                                     * np.float32(vscale))
    x["gamma"] = (x["gamma"] * np.float32(30.0)).astype(np.float32)
    x["S0"] = (x["S0"] * np.float32(vscale)).astype(np.float32)
    o, S = run(x, n)
    o_ref, S_ref = frame_forward(x["q"], x["k"], x["v"], x["gamma"], x["g"], n, x["S0"])
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(f"frame, repeated keys, gamma x30, v x {vscale:g}", o, S, o_ref, S_ref)
