"""Seeded synthetic inputs for the gated delta rule workloads.

This module only draws random numbers and shapes them; it contains none of the
recurrence's arithmetic.  Both the GPU path (through its tests and bench) and
the CPU oracle consume the arrays it returns, so the two sides always see the
same values.

Recipe (one generator per tensor, numpy PCG64, seed = 1000 * workload_id +
tensor_index, tensor order q, k, v, beta, g, S0):

* values are drawn in float32;
* q and k are L2-normalised per token over the key dimension in float32 (the
  pages normalise keys by convention: "Gated DeltaNet: Householder
  Transitions..." explainer and the video-delta-rule post, Preliminaries);
* q, k, v are then rounded to the I/O dtype with round-to-nearest-even;
* beta = sigmoid(N(0,1)); the gate is the log-decay g = log(alpha) in float32;
* Gated DeltaNet-2 workloads add an erase gate b [B,H,T,d_k] and a write gate
  w [B,H,T,d_v], each sigmoid(N(0,1)) (tensor indices 6 and 7; beta is then unused);
* the state is always float32.

The workloads mirror the shapes the pages use for their 1.3B training setup
(16 heads, d_k = d_v = 128, 4K sequence) plus a per-channel-decay, a long-context,
a decode and a Gated Delta Product shape (keys, values and betas per substep).  Every array is returned as float32 holding values that are
exactly representable in the I/O dtype; ``to_bf16_bits`` gives the raw bf16 bit
pattern for upload.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CHUNK = 64


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic workload."""

    wid: int
    name: str
    B: int
    H: int
    T: int
    d_k: int
    d_v: int
    io_dtype: str  # "f32" or "bf16"
    gate: str  # "scalar", "channel" or "gdn2" (channel decay, erase gate b and write gate w)
    g_dist: tuple  # ("uniform", lo, hi) or ("neg_softplus", scale)
    s0_std: float  # 0.0 means a zero initial state
    decode: bool = False
    steps: int = 1
    nh: int = 1  # substeps per token (Gated Delta Product); 1 = Gated DeltaNet
    note: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.B * self.T


WORKLOADS = {
    1: Workload(1, "tiny_f32", 1, 1, 256, 64, 64, "f32", "scalar", ("uniform", -0.1, -0.001), 0.0,
                note="tiny fp32 gated delta rule"),
    2: Workload(2, "gdn_bf16_train", 4, 16, 4096, 128, 128, "bf16", "scalar", ("neg_softplus", 0.05), 0.0,
                note="GDN bf16 training shape"),
    3: Workload(3, "kda_bf16", 2, 16, 8192, 128, 128, "bf16", "channel", ("neg_softplus", 0.05), 0.0,
                note="per-channel (KDA-style) decay"),
    4: Workload(4, "long_ctx_carried", 1, 32, 65536, 128, 128, "bf16", "scalar", ("uniform", -0.02, -0.0005), 0.02,
                note="long single sequence with carried state"),
    5: Workload(5, "decode", 256, 32, 1, 128, 128, "bf16", "scalar", ("uniform", -0.1, -0.001), 0.02,
                decode=True, steps=64, note="recurrent decode step, 64 steps"),
    6: Workload(6, "gdp_bf16", 4, 16, 2048, 128, 128, "bf16", "scalar", ("neg_softplus", 0.05), 0.0,
                nh=2, note="Gated Delta Product, 2 substeps per token (4096 substeps per sequence)"),
    7: Workload(7, "gdn2_bf16", 2, 16, 8192, 128, 128, "bf16", "gdn2", ("neg_softplus", 0.05), 0.0,
                note="Gated DeltaNet-2: per-channel decay, erase gate b and write gate w"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    # NaN stays NaN (keep a quiet-NaN payload in the top half)
    nan = np.isnan(x)
    out = rounded.astype(np.uint32).view(np.float32).copy()
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _rng(wid: int, tensor_index: int, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * wid + tensor_index + 7919 * salt))


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _cast_io(x: np.ndarray, io_dtype: str) -> np.ndarray:
    return round_to_bf16(x) if io_dtype == "bf16" else x.astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _gate(rng: np.random.Generator, shape, g_dist) -> np.ndarray:
    if g_dist[0] == "uniform":
        return rng.uniform(g_dist[1], g_dist[2], size=shape).astype(np.float32)
    if g_dist[0] == "neg_softplus":
        z = rng.standard_normal(size=shape, dtype=np.float32).astype(np.float64)
        return (-np.logaddexp(0.0, z) * g_dist[1]).astype(np.float32)
    raise ValueError(g_dist)


def make_inputs(w: Workload, *, B=None, H=None, T=None, salt: int = 0) -> dict:
    """Draw one input set for workload ``w``; B, H, T may be overridden (smaller
    parity cases keep the workload's distributions).  ``salt`` selects another
    independent set (used to rotate input sets when timing, and for decode steps).

    Returns float32 arrays: q, k [B,H,T,d_k]; v [B,H,T,d_v]; beta [B,H,T];
    g [B,H,T] (scalar gate) or [B,H,T,d_k] (channel gate); S0 [B,H,d_v,d_k] or None.
    With ``w.nh > 1`` (Gated Delta Product) k, v and beta carry a substep axis:
    k [B,H,T,n_h,d_k], v [B,H,T,n_h,d_v], beta [B,H,T,n_h]; q and g stay per token.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    dk, dv = w.d_k, w.d_v
    sub = (B, H, T) if w.nh == 1 else (B, H, T, w.nh)
    q = _rng(w.wid, 0, salt).standard_normal(size=(B, H, T, dk), dtype=np.float32)
    k = _rng(w.wid, 1, salt).standard_normal(size=sub + (dk,), dtype=np.float32)
    v = _rng(w.wid, 2, salt).standard_normal(size=sub + (dv,), dtype=np.float32)
    beta = _sigmoid(_rng(w.wid, 3, salt).standard_normal(size=sub, dtype=np.float32))
    gshape = (B, H, T) if w.gate == "scalar" else (B, H, T, dk)
    g = _gate(_rng(w.wid, 4, salt), gshape, w.g_dist)
    extra = {}
    if w.gate == "gdn2":  # erase gate b [B,H,T,d_k], write gate w [B,H,T,d_v], both sigmoid(N(0,1))
        extra["b"] = _sigmoid(_rng(w.wid, 6, salt).standard_normal(size=(B, H, T, dk), dtype=np.float32))
        extra["w"] = _sigmoid(_rng(w.wid, 7, salt).standard_normal(size=(B, H, T, dv), dtype=np.float32))
    S0 = None
    if w.s0_std > 0.0:
        S0 = (_rng(w.wid, 5, salt).standard_normal(size=(B, H, dv, dk), dtype=np.float32)
              * np.float32(w.s0_std)).astype(np.float32)
    q = _cast_io(_l2_normalise(q), w.io_dtype)
    k = _cast_io(_l2_normalise(k), w.io_dtype)
    v = _cast_io(v, w.io_dtype)
    out = {"q": q, "k": k, "v": v, "beta": beta, "g": g, "S0": S0}
    out.update(extra)
    return out


def make_raw_inputs(w: Workload, *, B=None, H=None, T=None, salt: int = 0, head_params: str = "plain") -> dict:
    """The raw draws that ``make_inputs`` turns into q, k, beta and g, for a scalar-gate
    workload with the ("neg_softplus", scale) gate: q_raw, k_raw [B,H,T,d_k] (N(0,1),
    rounded to the I/O dtype but NOT normalised), v [B,H,T,d_v], dt and beta_logit [B,H,T]
    (N(0,1)), and per-head A_log, dt_bias [H].  The same generators as ``make_inputs``.

    head_params "plain": A_log = log(scale), dt_bias = 0, so that -exp(A_log) softplus(dt +
    dt_bias) is the workload's g; "varied": A_log = log(scale) + U(-1, 1) and dt_bias ~
    N(0, 0.5^2) per head (tensor index 8).
    """
    assert w.gate == "scalar" and w.g_dist[0] == "neg_softplus" and w.nh == 1
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    dk, dv = w.d_k, w.d_v
    q = _rng(w.wid, 0, salt).standard_normal(size=(B, H, T, dk), dtype=np.float32)
    k = _rng(w.wid, 1, salt).standard_normal(size=(B, H, T, dk), dtype=np.float32)
    v = _rng(w.wid, 2, salt).standard_normal(size=(B, H, T, dv), dtype=np.float32)
    beta_logit = _rng(w.wid, 3, salt).standard_normal(size=(B, H, T), dtype=np.float32)
    dt = _rng(w.wid, 4, salt).standard_normal(size=(B, H, T), dtype=np.float32)
    A_log = np.full(H, np.log(w.g_dist[1]), dtype=np.float32)
    dt_bias = np.zeros(H, dtype=np.float32)
    if head_params == "varied":
        r = _rng(w.wid, 8, salt)
        A_log = (A_log + r.uniform(-1.0, 1.0, size=H)).astype(np.float32)
        dt_bias = (0.5 * r.standard_normal(size=H)).astype(np.float32)
    return {"q_raw": _cast_io(q, w.io_dtype), "k_raw": _cast_io(k, w.io_dtype), "v": _cast_io(v, w.io_dtype),
            "dt": dt, "beta_logit": beta_logit, "A_log": A_log, "dt_bias": dt_bias}


FRAME_WORKLOAD = dict(wid=8, name="frame_bf16", B=1, H=16, T=16384, frame_len=1024, d_k=128, d_v=128,
                      note="frame-level implicit update: 16 frames of 1024 tokens (video-like)")


def make_frame_inputs(*, B=1, H=16, T=16384, frame_len=1024, d_k=128, d_v=128, channel=True, salt: int = 0,
                      s0_std: float = 0.0) -> dict:
    """Inputs of the frame-level implicit update (wid 8): q, k ~ N(0,1) L2-normalised and v ~
    N(0,1), all rounded to bf16; writing strengths gamma = s e^z with s = d_k / frame_len (the
    post's suggested scale, old state and frame about equal) and z ~ N(0, 0.5^2); the log
    forget gate of each frame ~ U(-0.2, -0.01), per key channel (or one per frame).
    Returns float32 arrays: q, k [B,H,T,d_k]; v [B,H,T,d_v]; gamma [B,H,T]; g [B,H,F(,d_k)];
    S0 [B,H,d_v,d_k] or None."""
    wid = 8
    F = (T + frame_len - 1) // frame_len
    q = _rng(wid, 0, salt).standard_normal(size=(B, H, T, d_k), dtype=np.float32)
    k = _rng(wid, 1, salt).standard_normal(size=(B, H, T, d_k), dtype=np.float32)
    v = _rng(wid, 2, salt).standard_normal(size=(B, H, T, d_v), dtype=np.float32)
    z = _rng(wid, 3, salt).standard_normal(size=(B, H, T), dtype=np.float32)
    gamma = (np.float32(d_k / frame_len) * np.exp(np.float32(0.5) * z)).astype(np.float32)
    g = _rng(wid, 4, salt).uniform(-0.2, -0.01, size=(B, H, F, d_k) if channel else (B, H, F)).astype(np.float32)
    S0 = None
    if s0_std > 0.0:
        S0 = (_rng(wid, 5, salt).standard_normal(size=(B, H, d_v, d_k), dtype=np.float32)
              * np.float32(s0_std)).astype(np.float32)
    return {"q": round_to_bf16(_l2_normalise(q)), "k": round_to_bf16(_l2_normalise(k)), "v": round_to_bf16(v),
            "gamma": gamma, "g": g, "S0": S0}


def make_decode_inputs(w: Workload, step: int, *, N=None, H=None) -> dict:
    """Fresh per-step decode inputs (q, k [N,H,d_k]; v [N,H,d_v]; beta, g [N,H]
    or g [N,H,d_k]).  Step ``s`` uses salt ``s + 1``; the initial state comes
    from ``make_decode_state``."""
    N = w.B if N is None else N
    H = w.H if H is None else H
    x = make_inputs(w, B=N, H=H, T=1, salt=step + 1)
    out = {"q": x["q"][:, :, 0], "k": x["k"][:, :, 0], "v": x["v"][:, :, 0],
           "beta": x["beta"][:, :, 0], "g": x["g"][:, :, 0]}
    return {key: np.ascontiguousarray(val) for key, val in out.items()}


def make_decode_state(w: Workload, *, N=None, H=None) -> np.ndarray:
    """Initial decode state S [N,H,d_v,d_k] ~ s0_std * N(0,1), float32."""
    N = w.B if N is None else N
    H = w.H if H is None else H
    return (_rng(w.wid, 5).standard_normal(size=(N, H, w.d_v, w.d_k), dtype=np.float32)
            * np.float32(w.s0_std)).astype(np.float32)
