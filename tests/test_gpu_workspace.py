"""Parity of the per-chunk quantities that the two-kernel path's UT pass writes, against the
oracle's chunk form (white box: the test decodes the workspace records).

The end-to-end tests check o and the final state.  These compare the intermediate products of
the chunk-local transform with the fp64 oracle (oracle.chunk_transform, oracle.chunk_scores)
directly, chunk by chunk, including a ragged last chunk:
  scalar gate: A (the local scores), T = (I + diag(beta) L)^{-1} diag(beta) (the UT
    transform), e^{G_l}, e^{G_C - G_l} and e^{G_C};
  per-channel gate: A, T, K e^G, Q e^G, K e^{G_C - G} and e^{G_C} per key channel;
  fused input preparation: A, T and the per-token factors with the raw rows' inverse norms
    folded in;
  Gated DeltaNet-2: A, T = (I + M)^{-1} (oracle.gdn2_chunk_transform), the erase-side copy
    (b (.) k) e^G, Q e^G, K e^{G_C - G} and e^{G_C};
  Gated Delta Product: the scalar-gate records over the virtual sequence of substeps.

Record layout per (sequence, chunk), fp16 unless noted (C = 64):
  A^T (row m holds A[l][m]) without its all-zero 32x32 block (rows 32.., columns ..31): rows
    0..31 at full width, then rows 32..63 at columns 32..63, in 8-half pieces (3072 halfs);
  T, column m of each row stored at position pperm(m) inside its 32-column block, without its
    all-zero block (rows ..31, columns 32..): rows 0..31 at columns 0..31, then rows 32..63
    at full width (3072 halfs);
  scalar gate: fp32 e^{G_l} [C], e^{G_C - G_l} [C], e^{G_C}, 15 zeros;
  fused preparation: fp32 e^{G_l}/||k_l|| [C], e^{G_C - G_l}/||k_l|| [C], e^{G_C}, 15 zeros,
    e^{G_l}/||q_l|| [C];
  per-channel gate: K e^G, Q e^G, K e^{G_C - G} [C][d_k] each, then fp32 e^{G_C} [d_k].
Tokens past the end of a sequence enter the kernels as identity tokens (k = q = 0, g = 0,
beta = 0), so a ragged chunk's records hold the oracle's shorter chunk in their leading rows
and columns and zeros elsewhere (the factors repeat e^{G_C} past the end; Gated DeltaNet-2's
T = N^{-1} has ones on its diagonal there).

Bars.  The fp32 factors: 2e-6 relative (the kernels' exponential is accurate to a few ulp).
The fp16 matrices: max |gpu - oracle| / max |oracle| per chunk below 4e-3.  The stored value
is rounded to fp16 (2^-11 relative), and it is formed from fp16 operands (q and k exact, the
decay factors rounded) with fp32 accumulation: a few fp16 ulps of the largest element.
Measured on MI355X: at most 7.7e-4 (A at d_k = 64), 3.1e-4 (T), 6.3e-4 (the copies).
"""
import dataclasses

import numpy as np
import pytest

import gdr_synth
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gated_delta_rule_15_amd as gdr  # noqa: E402
from gated_delta_rule_15_amd._binding import GDR_BF16, GDR_GATE_CHANNEL, GDR_GATE_SCALAR  # noqa: E402

DEV = torch.device("cuda:0")
C = 64
TOL_F16 = 4e-3
TOL_F32 = 2e-6


def _pperm(m):
    return (m & ~31) | (((m >> 2) & 3) << 3) | (((m >> 4) & 1) << 2) | (m & 3)


PPERM = np.array([_pperm(m) for m in range(C)])


def _dev(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def _rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _records(wid, T, dk, gate_code):
    w = dataclasses.replace(gdr_synth.WORKLOADS[wid], d_k=dk, d_v=dk)
    x = gdr_synth.make_inputs(w, B=1, H=2, T=T)
    nbytes = gdr.chunk_fwd_workspace_size(1, 2, T, dk, dk, GDR_BF16, gate_code)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    gdr.chunk_fwd(_dev(x["q"], True), _dev(x["k"], True), _dev(x["v"], True), _dev(x["g"]), _dev(x["beta"]),
                  workspace=ws)
    torch.cuda.synchronize()
    nC = (T + C - 1) // C
    raw = ws.cpu().numpy()
    stride = nbytes // (2 * nC)
    return x, raw, stride, nC


def _f16(raw, byte_off, n):
    return raw[byte_off:byte_off + 2 * n].view(np.float16).astype(np.float64)


def _f32(raw, byte_off, n):
    return raw[byte_off:byte_off + 4 * n].view(np.float32).astype(np.float64)


TRI = 3 * C * C // 4          # halfs of one compact triangular matrix
FACTORS = 4 * TRI              # byte offset of the fp32 factor table (and of the KDA copies)


def _expand(flat, upper_zero):
    """A compact triangular matrix back to C x C, its left-out 32x32 block zero.  upper_zero:
    the block left out is rows 0..31 x columns 32..63 (T), else rows 32..63 x columns 0..31 (A^T)."""
    M = np.zeros((C, C))
    if upper_zero:
        M[:32, :32] = flat[:1024].reshape(32, 32)
        M[32:, :] = flat[1024:].reshape(32, 64)
    else:
        M[:32, :] = flat[:2048].reshape(32, 64)
        M[32:, 32:] = flat[2048:].reshape(32, 32)
    return M


def _check_at_t(rec, base, A_ref, T_ref, Cr, label, pad_diag=0.0):
    """A and T of one record against the oracle's leading Cr x Cr blocks.  Past the end of the
    sequence T holds pad_diag on its diagonal and zeros elsewhere: 0 where T carries diag(beta)
    (beta = 0 there), 1 for Gated DeltaNet-2's T = N^{-1}."""
    At = _expand(_f16(rec, base, TRI), upper_zero=False)
    Tp = _expand(_f16(rec, base + 2 * TRI, TRI), upper_zero=True)
    A = At.T
    Tm = Tp[:, PPERM]  # logical column m from its stored position
    eA = _rel(A[:Cr, :Cr], A_ref)
    eT = _rel(Tm[:Cr, :Cr], T_ref)
    print(f"{label}: e_A {eA:.2e} e_T {eT:.2e}")
    assert eA < TOL_F16 and eT < TOL_F16, label
    # structural zeros: above the diagonal, and every row or column of a padded token
    assert np.all(np.triu(A, 1) == 0.0) and np.all(np.triu(Tm, 1) == 0.0), label
    assert np.all(A[Cr:] == 0.0) and np.all(A[:, Cr:] == 0.0), label
    pad = np.zeros((C, C))
    pad[np.arange(Cr, C), np.arange(Cr, C)] = pad_diag
    assert np.all(Tm[Cr:] == pad[Cr:]) and np.all(Tm[:, Cr:] == pad[:, Cr:]), label


@pytest.mark.parametrize("T", [64, 100, 200])
@pytest.mark.parametrize("dk", [128, 64])
def test_ut_records_scalar_gate(T, dk):
    """UT transform of the scalar gate: A, T and the decay factors of every chunk."""
    x, raw, stride, nC = _records(2, T, dk, GDR_GATE_SCALAR)
    for h in range(2):
        for c in range(nC):
            s0, s1 = c * C, min(T, (c + 1) * C)
            Cr = s1 - s0
            Q, K = x["q"][0, h, s0:s1], x["k"][0, h, s0:s1]
            g, beta = x["g"][0, h, s0:s1], x["beta"][0, h, s0:s1]
            tr = oracle.chunk_transform(K, g, beta)
            A_ref, _ = oracle.chunk_scores(Q, K, g)
            base = (h * nC + c) * stride
            label = f"scalar d_k={dk} T={T} head {h} chunk {c}"
            _check_at_t(raw, base, A_ref, tr["T"], Cr, label)
            f = _f32(raw, base + FACTORS, 144)
            lam = tr["lam"]
            eg = np.array([lam(1, l) for l in range(1, Cr + 1)])
            er = np.array([lam(l + 1, Cr) for l in range(1, Cr + 1)])
            lamC = float(tr["lam_C"])
            assert _rel(f[:Cr], eg) < TOL_F32, label
            assert _rel(f[64:64 + Cr], er) < TOL_F32, label
            assert abs(f[128] - lamC) / lamC < TOL_F32, label
            # past the end: g = 0, so e^{G_l} stays at e^{G_C} and e^{G_C - G_l} at 1
            assert np.all(np.abs(f[Cr:64] - lamC) <= TOL_F32 * lamC), label
            assert np.all(np.abs(f[64 + Cr:128] - 1.0) <= TOL_F32), label
            assert np.all(f[129:144] == 0.0), label


@pytest.mark.parametrize("T", [64, 100])
@pytest.mark.parametrize("dk", [128, 64])
def test_ut_records_channel_gate(T, dk):
    """UT pass of the per-channel gate: A, T, the decayed copies and e^{G_C} per channel."""
    x, raw, stride, nC = _records(3, T, dk, GDR_GATE_CHANNEL)
    for h in range(2):
        for c in range(nC):
            s0, s1 = c * C, min(T, (c + 1) * C)
            Cr = s1 - s0
            Q, K = x["q"][0, h, s0:s1], x["k"][0, h, s0:s1]
            g, beta = x["g"][0, h, s0:s1], x["beta"][0, h, s0:s1]
            tr = oracle.chunk_transform(K, g, beta)
            A_ref, Q_left = oracle.chunk_scores(Q, K, g)
            base = (h * nC + c) * stride
            label = f"channel d_k={dk} T={T} head {h} chunk {c}"
            _check_at_t(raw, base, A_ref, tr["T"], Cr, label)
            off = base + FACTORS
            copies = {"K e^G": tr["K_left"], "Q e^G": Q_left, "K e^(G_C-G)": tr["K_right"]}
            for i, (name, ref) in enumerate(copies.items()):
                got = _f16(raw, off + i * 2 * C * dk, C * dk).reshape(C, dk)
                e = _rel(got[:Cr], ref)
                print(f"{label}: e[{name}] {e:.2e}")
                assert e < TOL_F16, (label, name)
                assert np.all(got[Cr:] == 0.0), (label, name)
            fe = _f32(raw, off + 3 * 2 * C * dk, dk)
            assert _rel(fe, np.asarray(tr["lam_C"])) < TOL_F32, label


@pytest.mark.parametrize("T", [64, 100])
@pytest.mark.parametrize("dk", [128, 64])
def test_ut_records_fused_prep(T, dk):
    """UT pass with the fused input preparation: A and T of the prepared inputs, and the state
    pass's per-token factors with the inverse norms of the raw rows folded in: e^{G_l}/||k_l||,
    e^{G_C - G_l}/||k_l||, e^{G_C} and e^{G_l}/||q_l|| (the state pass multiplies the raw rows'
    products by them)."""
    w = dataclasses.replace(gdr_synth.WORKLOADS[2], d_k=dk, d_v=dk)
    r = gdr_synth.make_raw_inputs(w, B=1, H=2, T=T, head_params="varied")
    nbytes = gdr.chunk_fwd_fused_prep_workspace_size(1, 2, T, dk, dk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    gdr.chunk_fwd_fused_prep(_dev(r["q_raw"], True), _dev(r["k_raw"], True), _dev(r["v"], True), _dev(r["dt"]),
                             _dev(r["A_log"]), _dev(r["dt_bias"]), _dev(r["beta_logit"]), workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    nC = (T + C - 1) // C
    stride = nbytes // (2 * nC)
    q, k, g, beta = oracle.prepare_inputs(r["q_raw"], r["k_raw"], r["dt"], r["A_log"], r["dt_bias"], r["beta_logit"])
    # the normalisation's inverse norms, 1 / max(||x_raw||, 1e-6), of the rows the kernel read
    inv = {n: 1.0 / np.maximum(np.linalg.norm(np.asarray(r[n], np.float64), axis=-1), 1e-6) for n in ("q_raw", "k_raw")}
    for h in range(2):
        for c in range(nC):
            s0, s1 = c * C, min(T, (c + 1) * C)
            Cr = s1 - s0
            Q, K = q[0, h, s0:s1], k[0, h, s0:s1]
            gc, bc = g[0, h, s0:s1], beta[0, h, s0:s1]
            tr = oracle.chunk_transform(K, gc, bc)
            A_ref, _ = oracle.chunk_scores(Q, K, gc)
            base = (h * nC + c) * stride
            label = f"prep d_k={dk} T={T} head {h} chunk {c}"
            _check_at_t(raw, base, A_ref, tr["T"], Cr, label)
            f = _f32(raw, base + FACTORS, 208)
            lam = tr["lam"]
            eg = np.array([lam(1, l) for l in range(1, Cr + 1)])
            er = np.array([lam(l + 1, Cr) for l in range(1, Cr + 1)])
            lamC = float(tr["lam_C"])
            ik, iq = inv["k_raw"][0, h, s0:s1], inv["q_raw"][0, h, s0:s1]
            assert _rel(f[:Cr], eg * ik) < TOL_F32, label
            assert _rel(f[64:64 + Cr], er * ik) < TOL_F32, label
            assert abs(f[128] - lamC) / lamC < TOL_F32, label
            assert np.all(f[129:144] == 0.0), label
            assert _rel(f[144:144 + Cr], eg * iq) < TOL_F32, label
            # past the end the rows are zero (inverse norm 1e6): the factors only ever multiply
            # products with those zero rows
            assert np.all(np.abs(f[Cr:64] - 1e6 * lamC) <= 1e-5 * 1e6 * lamC), label
            assert np.all(np.abs(f[144 + Cr:208] - 1e6 * lamC) <= 1e-5 * 1e6 * lamC), label


@pytest.mark.parametrize("T", [64, 100])
@pytest.mark.parametrize("dk", [128, 64])
def test_ut_records_gdn2(T, dk):
    """UT pass of Gated DeltaNet-2 against the oracle's chunk form (oracle.gdn2_chunk_transform):
    A, T = (I + M)^{-1} (no beta: the erase gate sits in the row operand), the erase-side copy
    (b (.) k) e^G in the K e^G slot, Q e^G, K e^{G_C - G} and e^{G_C}."""
    w = dataclasses.replace(gdr_synth.WORKLOADS[7], d_k=dk, d_v=dk)
    x = gdr_synth.make_inputs(w, B=1, H=2, T=T)
    nbytes = gdr.gdn2_chunk_fwd_workspace_size(1, 2, T, dk, dk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    gdr.gdn2_chunk_fwd(_dev(x["q"], True), _dev(x["k"], True), _dev(x["v"], True), _dev(x["g"]), _dev(x["b"]),
                       _dev(x["w"]), workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    nC = (T + C - 1) // C
    stride = nbytes // (2 * nC)
    for h in range(2):
        for c in range(nC):
            s0, s1 = c * C, min(T, (c + 1) * C)
            Cr = s1 - s0
            Q, K = x["q"][0, h, s0:s1], x["k"][0, h, s0:s1]
            g, b = x["g"][0, h, s0:s1], x["b"][0, h, s0:s1]
            tr = oracle.gdn2_chunk_transform(K, b * K, g)
            A_ref, Q_left = oracle.chunk_scores(Q, K, g)
            base = (h * nC + c) * stride
            label = f"gdn2 d_k={dk} T={T} head {h} chunk {c}"
            _check_at_t(raw, base, A_ref, tr["T_inv"], Cr, label, pad_diag=1.0)
            off = base + FACTORS
            copies = {"E e^G": tr["E_left"], "Q e^G": Q_left, "K e^(G_C-G)": tr["K_right"]}
            for i, (name, ref) in enumerate(copies.items()):
                got = _f16(raw, off + i * 2 * C * dk, C * dk).reshape(C, dk)
                e = _rel(got[:Cr], ref)
                print(f"{label}: e[{name}] {e:.2e}")
                assert e < TOL_F16, (label, name)
                assert np.all(got[Cr:] == 0.0), (label, name)
            fe = _f32(raw, off + 3 * 2 * C * dk, dk)
            assert _rel(fe, np.asarray(tr["lam_C"])) < TOL_F32, label


@pytest.mark.parametrize("T,nh", [(22, 3), (43, 3), (40, 2)])
def test_ut_records_gdp(T, nh):
    """UT pass of the Gated Delta Product, which runs the scalar-gate records over the virtual
    sequence of T n_h steps: against oracle.chunk_transform / chunk_scores on the page's
    mapping (oracle.gdp_as_virtual_gdn: decay on the first substep, q on the last)."""
    dk = 128
    w = dataclasses.replace(gdr_synth.WORKLOADS[6], nh=nh)
    x = gdr_synth.make_inputs(w, B=1, H=2, T=T)
    nbytes = gdr.gdp_chunk_fwd_workspace_size(1, 2, T, nh, dk, dk)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    gdr.gdp_chunk_fwd(_dev(x["q"], True), _dev(x["k"], True), _dev(x["v"], True), _dev(x["g"]), _dev(x["beta"]),
                      workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    qv, kv, _, gv, bv, _ = oracle.gdp_as_virtual_gdn(x["q"], x["k"], x["v"], x["g"], x["beta"])
    Tv = T * nh
    nC = (Tv + C - 1) // C
    stride = nbytes // (2 * nC)
    for h in range(2):
        for c in range(nC):
            s0, s1 = c * C, min(Tv, (c + 1) * C)
            Cr = s1 - s0
            Q, K = qv[0, h, s0:s1], kv[0, h, s0:s1]
            g, beta = gv[0, h, s0:s1], bv[0, h, s0:s1]
            tr = oracle.chunk_transform(K, g, beta)
            A_ref, _ = oracle.chunk_scores(Q, K, g)
            base = (h * nC + c) * stride
            label = f"gdp n_h={nh} T={T} head {h} chunk {c}"
            _check_at_t(raw, base, A_ref, tr["T"], Cr, label)
            f = _f32(raw, base + FACTORS, 144)
            lam = tr["lam"]
            assert _rel(f[:Cr], np.array([lam(1, l) for l in range(1, Cr + 1)])) < TOL_F32, label
            assert _rel(f[64:64 + Cr], np.array([lam(l + 1, Cr) for l in range(1, Cr + 1)])) < TOL_F32, label
            assert abs(f[128] - float(tr["lam_C"])) / float(tr["lam_C"]) < TOL_F32, label
