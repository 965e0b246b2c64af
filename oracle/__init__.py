"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Nothing on the product path imports this package: only ``tests/``, the smoke
check in ``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` do.
It shares no code with the HIP library and never touches the GPU.

Two independent fp64 implementations live here:

* ``recurrent_forward`` / ``decode_step`` -- the token-by-token recurrence in
  plain C (``gdr_oracle.c``), the definition the GPU path is judged against;
* ``chunked.chunked_forward`` -- the per-chunk algorithm of "Linear Attention,
  Visualized" (sections "Gated DeltaNet (GDN)" and "Reuse GLA and GDN"),
  written in numpy, used only to cross-check the recurrence (every chunk size
  gives the exact result, section "Cost").
* ``gdp_forward`` -- Gated Delta Product token by token (section "Gated Delta
  Product (GDP)"), with the explicit n_h-substep update in the page's row
  notation, in C; and ``gdp_as_virtual_gdn``, the input mapping of section
  "GDP as GDN over a virtual sequence" that turns a GDP problem into a GDN one.
* ``prepare_inputs`` -- the step upstream of the path: unit-norm q and k (the
  pages' convention), beta = sigmoid(logit) in (0, 1), and Mamba-2's decay gate
  g = log a = -exp(A_log) softplus(dt + dt_bias) ("Linear Attention, Visualized",
  "Optional: Constructing the decay gate"), in numpy fp64.
* ``frame.frame_forward`` -- the frame-level implicit update of the video
  delta-rule post ("A Different Route"): per frame, S_t (I + G_t) = S_{t-1} D_t + C_t
  by a Cholesky factorisation and triangular solves, in numpy fp64.
* ``gdn2_forward`` -- Gated DeltaNet-2 token by token ("Gated DeltaNet-2, and the
  gate that was doing two jobs", section 2 "What decoupling actually means here"):
  KDA's decay with the scalar beta split into a key-side erase gate and a
  value-side write gate, in C.

Both are pinned by ``tests/test_oracle_*.py`` against closed forms, limits and
brute force that do not reuse them.  Parity of every function here is pinned;
absolute values at the full workload sizes are pinned only through these
functions themselves (the pages print no worked numbers).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
# GDR_ORACLE_LIBRARY names another build of the same source (the host-sanitizer test loads an
# AddressSanitizer / UndefinedBehaviorSanitizer build this way); it is used as it is.
_LIB = os.environ.get("GDR_ORACLE_LIBRARY") or os.path.join(_HERE, "libgdr_oracle.so")
_lock = threading.Lock()
_lib = None

GATE_SCALAR = 0
GATE_CHANNEL = 1


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (host only, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if "GDR_ORACLE_LIBRARY" not in os.environ and (
                    not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            lib.oracle_gdr_forward.argtypes = [ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, P, P, P, P, P, P, P, P, ctypes.c_int]
            lib.oracle_gdr_forward.restype = ctypes.c_int
            lib.oracle_gdr_decode_step.argtypes = [ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   P, P, P, P, P, P, P, ctypes.c_int]
            lib.oracle_gdr_decode_step.restype = ctypes.c_int
            lib.oracle_gdp_forward.argtypes = [ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, P, P, P, P, P, P, P, P, ctypes.c_int]
            lib.oracle_gdp_forward.restype = ctypes.c_int
            lib.oracle_gdn2_forward.argtypes = [ctypes.c_long, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                                P, P, P, P, P, P, P, P, P, ctypes.c_int]
            lib.oracle_gdn2_forward.restype = ctypes.c_int
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrent_forward(q, k, v, g, beta, S0=None, nthreads: int = 0):
    """Token recurrence in fp64.

    q, k [B,H,T,d_k]; v [B,H,T,d_v]; beta [B,H,T]; g [B,H,T] (scalar gate,
    log-decay) or [B,H,T,d_k] (channel gate); S0 [B,H,d_v,d_k] or None.
    Returns (o [B,H,T,d_v], S_T [B,H,d_v,d_k]) as float64.
    """
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    if g.shape == (B, H, T):
        gate = GATE_SCALAR
    elif g.shape == (B, H, T, dk):
        gate = GATE_CHANNEL
    else:
        raise ValueError(f"gate shape {g.shape} matches neither [B,H,T] nor [B,H,T,d_k]")
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(S0, dtype=np.float64)
        assert s0.shape == (B, H, dv, dk)
    o = np.empty((B, H, T, dv), dtype=np.float64)
    S = np.empty((B, H, dv, dk), dtype=np.float64)
    rc = _load().oracle_gdr_forward(B * H, T, dk, dv, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(s0), _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdr_forward failed ({rc})")
    return o, S


def decode_step(q, k, v, g, beta, S, nthreads: int = 0):
    """One recurrent step on resident states, fp64.

    q, k [N,H,d_k]; v [N,H,d_v]; beta [N,H]; g [N,H] or [N,H,d_k];
    S [N,H,d_v,d_k].  Returns (o [N,H,d_v], S_new) as float64 (S is not modified).
    """
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[-1]
    if g.shape == (N, H):
        gate = GATE_SCALAR
    elif g.shape == (N, H, dk):
        gate = GATE_CHANNEL
    else:
        raise ValueError(f"gate shape {g.shape}")
    Snew = np.array(S, dtype=np.float64, copy=True, order="C")
    assert Snew.shape == (N, H, dv, dk)
    o = np.empty((N, H, dv), dtype=np.float64)
    rc = _load().oracle_gdr_decode_step(N * H, dk, dv, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                        _ptr(beta), _ptr(Snew), _ptr(o), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdr_decode_step failed ({rc})")
    return o, Snew


def gdp_forward(q, k, v, g, beta, S0=None, nthreads: int = 0):
    """Gated Delta Product, token by token, fp64 ("Linear Attention, Visualized",
    section "Gated Delta Product (GDP)").

    q [B,H,T,d_k]; k [B,H,T,n_h,d_k]; v [B,H,T,n_h,d_v]; beta [B,H,T,n_h];
    g [B,H,T] (one log-decay per real token); S0 [B,H,d_v,d_k] or None.
    Returns (o [B,H,T,d_v], S_T [B,H,d_v,d_k]) as float64.
    """
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    B, H, T, dk = q.shape
    nh = k.shape[3]
    dv = v.shape[-1]
    assert k.shape == (B, H, T, nh, dk) and v.shape == (B, H, T, nh, dv)
    assert beta.shape == (B, H, T, nh) and g.shape == (B, H, T)
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(S0, dtype=np.float64)
        assert s0.shape == (B, H, dv, dk)
    o = np.empty((B, H, T, dv), dtype=np.float64)
    S = np.empty((B, H, dv, dk), dtype=np.float64)
    rc = _load().oracle_gdp_forward(B * H, T, nh, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(s0), _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdp_forward failed ({rc})")
    return o, S


def gdn2_forward(q, k, v, g, b, w, S0=None, nthreads: int = 0):
    """Gated DeltaNet-2 token recurrence, fp64.

    q, k, g, b [B,H,T,d_k] (g the per-channel log-decay, b the erase gate); v, w [B,H,T,d_v]
    (w the write gate); S0 [B,H,d_v,d_k] or None.  Returns (o [B,H,T,d_v], S_T) as float64.
    """
    q, k, v, g, b, w = map(_f32, (q, k, v, g, b, w))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == g.shape == b.shape == (B, H, T, dk) and w.shape == v.shape == (B, H, T, dv)
    s0 = None
    if S0 is not None:
        s0 = np.ascontiguousarray(S0, dtype=np.float64)
        assert s0.shape == (B, H, dv, dk)
    o = np.empty((B, H, T, dv), dtype=np.float64)
    S = np.empty((B, H, dv, dk), dtype=np.float64)
    rc = _load().oracle_gdn2_forward(B * H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                                     _ptr(s0), _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gdn2_forward failed ({rc})")
    return o, S


def prepare_inputs(q_raw, k_raw, dt, A_log, dt_bias, beta_logit, eps: float = 1e-6):
    """Inputs of the gated delta rule from raw projections, fp64.

    * q = q_raw / max(||q_raw||_2, eps), k likewise, per token over d_k: the pages take
      keys (and queries) L2-normalised by convention ("Gated DeltaNet: Householder
      Transitions...", video-delta-rule post, Preliminaries); eps only keeps a zero vector
      at zero.
    * beta = 1 / (1 + exp(-beta_logit)): the pages require 0 < beta <= 1; the logistic map
      is the plain way to get there.
    * g = log a = -exp(A_log[h]) * softplus(dt + dt_bias[h]), softplus(x) = log(1 + e^x):
      "Linear Attention, Visualized", section "Mamba-2: input-dependent scalar decay",
      "Optional: Constructing the decay gate" (a_t = exp(-lambda Delta_t), lambda =
      e^{A_log}, Delta_t = softplus(dt_t + b_Delta)).

    q_raw, k_raw [B,H,T,d_k]; dt, beta_logit [B,H,T]; A_log, dt_bias [H].
    Returns (q, k, g, beta) as float64.
    """
    q_raw, k_raw, dt, beta_logit = (np.asarray(x, dtype=np.float64) for x in (q_raw, k_raw, dt, beta_logit))
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)

    def unit(x):
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return x / np.maximum(n, eps)

    lam = np.exp(A_log)[None, :, None]
    z = dt + dt_bias[None, :, None]
    softplus = np.logaddexp(0.0, z)
    g = -lam * softplus
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    return unit(q_raw), unit(k_raw), g, beta


def gdp_as_virtual_gdn(q, k, v, g, beta):
    """The mapping of section "GDP as GDN over a virtual sequence".

    Real token t and substep j (both 1-based on the page) become virtual step
    m = n_h (t - 1) + j, carrying (k, v, beta)_{t,j}; the decay a_t sits on the
    first substep (a = 1, i.e. log-decay 0, on the others) and the query q_t on
    the last (zero query on the others).  The GDN outputs to keep are those of
    virtual steps m = t n_h, i.e. indices n_h - 1, 2 n_h - 1, ... (0-based).

    Inputs as ``gdp_forward``; returns (q~, k~, v~, g~, beta~) of GDN shapes over
    T n_h steps and the 0-based indices of the kept outputs.
    """
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    B, H, T, nh, dk = k.shape
    dv = v.shape[-1]
    kt = k.reshape(B, H, T * nh, dk)
    vt = v.reshape(B, H, T * nh, dv)
    bt = beta.reshape(B, H, T * nh)
    gt = np.zeros((B, H, T, nh), dtype=np.float32)
    gt[..., 0] = g
    qt = np.zeros((B, H, T, nh, dk), dtype=np.float32)
    qt[..., nh - 1, :] = q
    keep = np.arange(T) * nh + (nh - 1)
    return qt.reshape(B, H, T * nh, dk), kt, vt, gt.reshape(B, H, T * nh), bt, keep


from .chunked import (chunk_scores, chunk_transform, chunked_forward, gdn2_chunk_transform,  # noqa: E402,F401
                      gdn2_chunked_forward)
from .frame import frame_forward  # noqa: E402,F401
