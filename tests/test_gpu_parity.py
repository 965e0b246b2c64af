"""GPU parity of libgdr against the fp64 CPU oracle (run on an MI355X).

Small cases span several chunks and a ragged tail and compare every element; the
full workload sizes run the GPU in the launch configuration the bench times and
compare sampled (batch, head) sequences, which the oracle computes independently
(sequences never interact).  Bars: tests/parity.py.
"""
import dataclasses

import numpy as np
import pytest

import gdr_synth
import oracle
from parity import TOL_BF16, TOL_F32, err_bf16_out, err_literal, report

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


def variant(wid, **kw):
    return dataclasses.replace(gdr_synth.WORKLOADS[wid], **kw)


def run_chunk(x, bf16, S0=None, **kw):
    o, S = gdr.chunk_fwd(dev(x["q"], bf16), dev(x["k"], bf16), dev(x["v"], bf16), dev(x["g"]), dev(x["beta"]),
                         dev(S0), **kw)
    torch.cuda.synchronize()
    return o, S


def check(name, o, S, o_ref, S_ref, bf16):
    eo, es, msg = report(name, host(o), o_ref, None if S is None else host(S), S_ref, bf16)
    print(msg)
    tol = TOL_BF16 if bf16 else TOL_F32
    assert eo <= tol and es <= tol, msg


# ----------------------------------------------------------------------------- decode
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 32), (64, 96)])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_decode_small(dk, dv, io, gate):
    w = variant(5, d_k=dk, d_v=dv, io_dtype=io, gate=gate)
    N, H, steps = 3, 2, 5
    st = gdr_synth.make_decode_state(w, N=N, H=H)
    state = dev(st)
    ref = st.astype(np.float64)
    bf16 = io == "bf16"
    for s in range(steps):
        d = gdr_synth.make_decode_inputs(w, s, N=N, H=H)
        o = gdr.decode_step(dev(d["q"], bf16), dev(d["k"], bf16), dev(d["v"], bf16), dev(d["g"]), dev(d["beta"]),
                            state)
        o_ref, ref = oracle.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], ref)
        torch.cuda.synchronize()
        eo = err_bf16_out(host(o), o_ref) if bf16 else err_literal(host(o), o_ref)
        assert eo <= (TOL_BF16 if bf16 else TOL_F32), (s, eo)
    es = err_literal(host(state), ref)
    assert es <= TOL_F32, es   # the state is fp32 in both I/O modes


@pytest.mark.parametrize("kind", ["identity", "exact_write", "reflection"])
def test_decode_special_values(kind):
    """g = 0 and beta = 0 (the identity: the state must come back bit for bit), beta = 1 (the
    exact write of v along k) and beta = 2 (a reflection, "A Swap Is a Reflection"), three
    steps each against the oracle."""
    w = variant(5)
    N, H, steps = 3, 2, 3
    st = gdr_synth.make_decode_state(w, N=N, H=H)
    state = dev(st)
    ref = st.astype(np.float64)
    for s in range(steps):
        d = gdr_synth.make_decode_inputs(w, s, N=N, H=H)
        if kind == "identity":
            d["g"][:] = 0.0
            d["beta"][:] = 0.0
        else:
            d["beta"][:] = 1.0 if kind == "exact_write" else 2.0
        o = gdr.decode_step(dev(d["q"], True), dev(d["k"], True), dev(d["v"], True), dev(d["g"]), dev(d["beta"]), state)
        o_ref, ref = oracle.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], ref)
        torch.cuda.synchronize()
        assert err_bf16_out(host(o), o_ref) <= TOL_BF16, (kind, s)
    assert err_literal(host(state), ref) <= TOL_F32
    if kind == "identity":
        assert torch.equal(state.cpu(), torch.from_numpy(st))


def test_decode_full_size_64_steps_sampled():
    """256 sequences x 32 heads, d = 128, 64 fresh-input steps on a 512 MiB state;
    48 sampled (sequence, head) states checked at every step against the oracle."""
    w = gdr_synth.WORKLOADS[5]
    N, H = w.B, w.H
    st = gdr_synth.make_decode_state(w)
    state = dev(st)
    rng = np.random.default_rng(5)
    pick = np.sort(rng.choice(N * H, size=48, replace=False))
    ni, hi = pick // H, pick % H
    ref = st[ni, hi][:, None].astype(np.float64)  # [48,1,dv,dk]
    worst = 0.0
    for s in range(w.steps):
        d = gdr_synth.make_decode_inputs(w, s)
        o = gdr.decode_step(dev(d["q"], True), dev(d["k"], True), dev(d["v"], True), dev(d["g"]), dev(d["beta"]),
                            state)
        sub = {kk: d[kk][ni, hi][:, None] for kk in d}
        o_ref, ref = oracle.decode_step(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], ref)
        torch.cuda.synchronize()
        eo = err_bf16_out(host(o)[ni, hi][:, None], o_ref)
        worst = max(worst, eo)
    es = err_literal(host(state)[ni, hi][:, None], ref)
    print(f"decode full size: worst e_o over 64 steps = {worst:.3e}, e_S = {es:.3e}")
    assert worst <= TOL_BF16 and es <= TOL_F32


# ----------------------------------------------------------------------------- chunk_fwd


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 32), (64, 64), (128, 256), (64, 96)])
@pytest.mark.parametrize("with_s0", [False, True])
def test_chunk_small_bf16(T, dk, dv, with_s0):
    w = variant(2, d_k=dk, d_v=dv)
    x = gdr_synth.make_inputs(w, B=2, H=2, T=T)
    S0 = (np.random.default_rng(T).standard_normal((2, 2, dv, dk)) * 0.05).astype(np.float32) if with_s0 else None
    o, S = run_chunk(x, True, S0)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"chunk bf16 T={T} dk={dk} dv={dv} s0={with_s0}", o, S, o_ref, S_ref, True)




def test_chunk_split_explicit_workspace_reused():
    """A caller-owned workspace, reused across calls of different sizes (its contents on
    entry do not matter)."""
    need = gdr.chunk_fwd_workspace_size(2, 2, 300, 128, 128)
    wsb = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    for T in (300, 70, 5):
        x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=2, H=2, T=T, salt=T)
        o, S = run_chunk(x, True, None, workspace=wsb)
        o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
        check(f"chunk, reused workspace T={T}", o, S, o_ref, S_ref, True)


@pytest.mark.parametrize("T", [1, 63, 100, 256])
@pytest.mark.parametrize("dv", [32, 64, 96])
def test_chunk_small_f32(T, dv):
    w = variant(1, d_v=dv)
    x = gdr_synth.make_inputs(w, B=1, H=3, T=T)
    S0 = (np.random.default_rng(T).standard_normal((1, 3, dv, 64)) * 0.05).astype(np.float32)
    o, S = run_chunk(x, False, S0)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"chunk f32 T={T} dv={dv}", o, S, o_ref, S_ref, False)


def test_chunk_workload1_tiny_f32():
    w = gdr_synth.WORKLOADS[1]
    x = gdr_synth.make_inputs(w)
    o, S = run_chunk(x, False, x["S0"])
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    check("workload 1 (tiny fp32)", o, S, o_ref, S_ref, False)


def _sampled_full(wid, nsample, seed, **kw):
    w = gdr_synth.WORKLOADS[wid]
    x = gdr_synth.make_inputs(w)
    o, S = run_chunk(x, True, x["S0"], **kw)
    rng = np.random.default_rng(seed)
    pick = np.sort(rng.choice(w.B * w.H, size=nsample, replace=False))
    bi, hi = pick // w.H, pick % w.H
    sub = {kk: (None if x[kk] is None else x[kk][bi, hi][None]) for kk in x}
    o_ref, S_ref = oracle.recurrent_forward(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], sub["S0"])
    o_s = o[torch.from_numpy(bi), torch.from_numpy(hi)][None]
    S_s = S[torch.from_numpy(bi), torch.from_numpy(hi)][None]
    return o_s, S_s, o_ref, S_ref


def test_chunk_workload2_full_size_sampled():
    """B=4, H=16, T=4096, d=128 bf16; 8 of the 64 sequences checked."""
    o, S, o_ref, S_ref = _sampled_full(2, 8, 2)
    check("workload 2 full size (8 sampled heads)", o, S, o_ref, S_ref, True)


def test_chunk_workload4_full_size_sampled():
    """B=1, H=32, T=65536, d=128 bf16 with a carried initial state; 2 heads checked."""
    o, S, o_ref, S_ref = _sampled_full(4, 2, 4)
    check("workload 4 full size (2 sampled heads)", o, S, o_ref, S_ref, True)


# ----------------------------------------------------------------------------- chunk_fwd, per-channel gate
@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 32), (64, 64), (128, 256), (64, 96)])
@pytest.mark.parametrize("with_s0", [False, True])
def test_chunk_kda_small(T, dk, dv, with_s0):
    w = variant(3, d_k=dk, d_v=dv)
    x = gdr_synth.make_inputs(w, B=2, H=2, T=T)
    S0 = (np.random.default_rng(T).standard_normal((2, 2, dv, dk)) * 0.05).astype(np.float32) if with_s0 else None
    o, S = run_chunk(x, True, S0)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"chunk kda T={T} dk={dk} dv={dv} s0={with_s0}", o, S, o_ref, S_ref, True)


@pytest.mark.parametrize("lo,hi", [(-3.0, -0.5), (-8.0, -0.01)])
def test_chunk_kda_strong_decay(lo, hi):
    """Per-channel log-decays far beyond the fp16 range of the in-block factors (the
    diagonal tiles take the exact path); mixed with weak channels so both paths meet."""
    w = variant(3, g_dist=("uniform", lo, hi))
    x = gdr_synth.make_inputs(w, B=1, H=2, T=200)
    x["g"][..., ::3] = x["g"][..., ::3] * 0.01  # every third channel decays slowly
    o, S = run_chunk(x, True)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    check(f"chunk kda strong decay U({lo},{hi})", o, S, o_ref, S_ref, True)


@pytest.mark.parametrize("wid", [2, 3])
def test_chunk_full_grid_small_T(wid):
    """B=4, H=16, d=128: 256 value tiles of 32 channels, the grid the state pass serves with two
    consumer waves per workgroup (smaller grids take 16-channel tiles); every sequence checked."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=4, H=16, T=150)
    S0 = (np.random.default_rng(wid).standard_normal((4, 16, 128, 128)) * 0.02).astype(np.float32)
    o, S = run_chunk(x, True, S0)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check(f"full grid, workload {wid} gate, T=150", o, S, o_ref, S_ref, True)




def test_chunk_kda_uniform_gate_matches_scalar_gate():
    """P9 on the GPU: a per-channel gate equal across channels gives the scalar-gate result."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=1, H=2, T=300)
    o1, S1 = run_chunk(x, True)
    xc = dict(x)
    xc["g"] = np.repeat(x["g"][..., None], x["q"].shape[-1], axis=-1).copy()
    o2, S2 = run_chunk(xc, True)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    check("kda with a uniform gate", o2, S2, o_ref, S_ref, True)
    check("scalar gate", o1, S1, o_ref, S_ref, True)


def test_chunk_workload3_full_size_sampled():
    """B=2, H=16, T=8192, d=128 bf16, per-channel gate; 2 of the 32 sequences checked."""
    o, S, o_ref, S_ref = _sampled_full(3, 2, 3)
    check("workload 3 full size (2 sampled heads)", o, S, o_ref, S_ref, True)


def test_chunk_kda_carried_state_split():
    w = variant(3, s0_std=0.02)
    x = gdr_synth.make_inputs(w, B=1, H=2, T=300)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    t0 = 140
    a = {kk: (vv if kk == "S0" else vv[:, :, :t0]) for kk, vv in x.items()}
    b = {kk: (None if kk == "S0" else vv[:, :, t0:]) for kk, vv in x.items()}
    oa, Sa = run_chunk(a, True, x["S0"])
    ob, Sb = gdr.chunk_fwd(dev(b["q"], True), dev(b["k"], True), dev(b["v"], True), dev(b["g"]), dev(b["beta"]), Sa)
    torch.cuda.synchronize()
    check(f"kda split at {t0}", torch.cat([oa, ob], dim=2), Sb, o_ref, S_ref, True)


def test_chunk_deterministic():
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=1, H=4, T=300)
    o1, S1 = run_chunk(x, True)
    o2, S2 = run_chunk(x, True)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_concurrent_calls_on_separate_streams():
    """Calls from several host threads, each on its own stream with its own buffers and
    workspace, give the results of the same calls made one after another (the library keeps
    no state between calls beyond per-device launch settings)."""
    import threading
    cases = [(2, 300, "scalar"), (3, 200, "channel"), (2, 129, "scalar"), (3, 64, "channel")]
    inputs = [gdr_synth.make_inputs(gdr_synth.WORKLOADS[wid], B=1, H=3, T=T, salt=i)
              for i, (wid, T, _) in enumerate(cases)]
    expect = [run_chunk(x, True) for x in inputs]
    got = [None] * len(cases)
    errors = []
    dev_in = [{key: dev(val, key in ("q", "k", "v")) for key, val in x.items() if val is not None} for x in inputs]
    torch.cuda.synchronize()

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            d = dev_in[i]
            with torch.cuda.stream(stream):
                for _ in range(3):
                    got[i] = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], stream=stream)
            stream.synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (o1, S1), (o2, S2) in zip(expect, got):
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_chunk_final_state_may_alias_initial_state():
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=1, H=2, T=130)
    S0 = (np.random.default_rng(1).standard_normal((1, 2, 128, 128)) * 0.05).astype(np.float32)
    s = dev(S0)
    o, S = run_chunk(x, True, None, final_state=None)  # warm-up, unrelated
    o, S = gdr.chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]), dev(x["beta"]), s,
                         final_state=s)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0)
    check("aliased state", o, s, o_ref, S_ref, True)


def test_chunk_empty_sequence_copies_state():
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[2], B=1, H=2, T=0)
    S0 = (np.random.default_rng(2).standard_normal((1, 2, 128, 128)) * 0.05).astype(np.float32)
    o, S = run_chunk(x, True, S0)
    assert o.numel() == 0 and torch.equal(S.cpu(), torch.from_numpy(S0))
    o, S = run_chunk(x, True, None)
    assert torch.count_nonzero(S) == 0


def test_chunk_carried_state_split():
    """chunk_fwd(x[:t0]) then chunk_fwd(x[t0:], S) matches the oracle on x, aligned and not."""
    x = gdr_synth.make_inputs(gdr_synth.WORKLOADS[4], B=1, H=2, T=500)
    o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    for t0 in (128, 200):
        a = {kk: (vv if kk == "S0" else vv[:, :, :t0]) for kk, vv in x.items()}
        b = {kk: (None if kk == "S0" else vv[:, :, t0:]) for kk, vv in x.items()}
        oa, Sa = run_chunk(a, True, x["S0"])
        ob, Sb = gdr.chunk_fwd(dev(b["q"], True), dev(b["k"], True), dev(b["v"], True), dev(b["g"]),
                               dev(b["beta"]), Sa)
        torch.cuda.synchronize()
        check(f"split at {t0}", torch.cat([oa, ob], dim=2), Sb, o_ref, S_ref, True)


def test_prefill_then_decode_handoff():
    """The chunked forward's final state feeds the decode step (P10 across the two paths)."""
    w = gdr_synth.WORKLOADS[2]
    x = gdr_synth.make_inputs(w, B=2, H=2, T=150)
    o, S = run_chunk(x, True)
    _, ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    wd = variant(5, B=2, H=2, g_dist=w.g_dist)
    for s in range(3):
        d = gdr_synth.make_decode_inputs(wd, s, N=2, H=2)
        od = gdr.decode_step(dev(d["q"], True), dev(d["k"], True), dev(d["v"], True), dev(d["g"]), dev(d["beta"]),
                             S)
        o_ref, ref = oracle.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], ref)
        torch.cuda.synchronize()
        assert err_bf16_out(host(od), o_ref) <= TOL_BF16
    assert err_literal(host(S), ref) <= TOL_BF16


# ----------------------------------------------------------------------------- full grid, d_k = 64
@pytest.mark.parametrize("mode", ["gdn", "kda", "gdn2", "gdp", "prep"])
def test_two_kernel_modes_full_grid_dk64(mode):
    """B=4, H=16, d_k=64, d_v=128: 256 value tiles of 32 channels, so every two-kernel mode runs
    its two-consumer-wave state kernel at d_k = 64; every sequence checked against the oracle."""
    B, H, T = 4, 16, 100
    if mode in ("gdn", "kda"):
        x = gdr_synth.make_inputs(variant(2 if mode == "gdn" else 3, d_k=64, d_v=128), B=B, H=H, T=T)
        o, S = run_chunk(x, True)
        o_ref, S_ref = oracle.recurrent_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    elif mode == "gdn2":
        x = gdr_synth.make_inputs(variant(7, d_k=64, d_v=128), B=B, H=H, T=T)
        o, S = gdr.gdn2_chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]), dev(x["b"]),
                                  dev(x["w"]))
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.gdn2_forward(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"])
    elif mode == "gdp":
        x = gdr_synth.make_inputs(variant(6, d_k=64, d_v=128, nh=2), B=B, H=H, T=T // 2)
        o, S = gdr.gdp_chunk_fwd(dev(x["q"], True), dev(x["k"], True), dev(x["v"], True), dev(x["g"]),
                                 dev(x["beta"]))
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.gdp_forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    else:
        r = gdr_synth.make_raw_inputs(variant(2, d_k=64, d_v=128), B=B, H=H, T=T, head_params="varied")
        o, S = gdr.chunk_fwd_fused_prep(dev(r["q_raw"], True), dev(r["k_raw"], True), dev(r["v"], True),
                                        dev(r["dt"]), dev(r["A_log"]), dev(r["dt_bias"]), dev(r["beta_logit"]))
        torch.cuda.synchronize()
        q, k, g, beta = oracle.prepare_inputs(r["q_raw"], r["k_raw"], r["dt"], r["A_log"], r["dt_bias"],
                                              r["beta_logit"])
        o_ref, S_ref = oracle.recurrent_forward(q, k, r["v"], g, beta)
    check(f"{mode} full grid d_k=64", o, S, o_ref, S_ref, True)
