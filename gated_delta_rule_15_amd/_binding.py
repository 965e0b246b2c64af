"""ctypes binding of libgdr (include/gdr.h): argument marshalling only.

PyTorch provides device memory and the HIP stream; every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is missing or a call fails, an
exception is raised.

Buffers the binding allocates (outputs, and the workspace when none is passed) are allocated
while the call's stream is torch's current stream, so torch's caching allocator orders their
reuse after the kernels enqueued on that stream.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
# GDR_LIBRARY names another build of the library (the host-sanitizer test loads one this way)
LIBRARY_PATH = os.environ.get("GDR_LIBRARY") or os.path.join(_PKG, "libgdr.so")

GDR_OK = 0
GDR_ERR_INVALID_ARG = 1
GDR_ERR_SHAPE = 2
GDR_ERR_DTYPE = 3
GDR_ERR_UNSUPPORTED = 4
GDR_ERR_WORKSPACE = 5
GDR_ERR_HIP = 6
GDR_BF16, GDR_F32 = 0, 1
GDR_GATE_SCALAR, GDR_GATE_CHANNEL = 0, 1

# every entry point include/gdr.h declares
EXPORTED_SYMBOLS = ("gdr_version", "gdr_status_string", "gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd",
                    "gdr_chunk_fwd_noalloc",
                    "gdr_chunk_fwd_fused_prep_workspace_size", "gdr_chunk_fwd_fused_prep",
                    "gdr_gdp_chunk_fwd_workspace_size", "gdr_gdp_chunk_fwd", "gdr_gdn2_chunk_fwd_workspace_size",
                    "gdr_gdn2_chunk_fwd", "gdr_frame_fwd_workspace_size", "gdr_frame_fwd", "gdr_decode_step")

_lock = threading.Lock()
_lib = None


class GdrError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_string(status)}")


def load_library():
    """Load libgdr.so (raises OSError with a build hint if it is missing)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIBRARY_PATH):
            raise OSError(f"{LIBRARY_PATH} not found: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIBRARY_PATH)
        i64, i32, P = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        sigs = {
            "gdr_version": (i32, []),
            "gdr_status_string": (ctypes.c_char_p, [i32]),
            "gdr_chunk_fwd_workspace_size": (i64, [i64, i64, i64, i32, i32, i32, i32]),
            "gdr_chunk_fwd": (i32, [i64, i64, i64, i32, i32, i32, i32] + [P] * 9 + [i64, P]),
            "gdr_chunk_fwd_noalloc": (i32, [i64, i64, i64, i32, i32, i32, i32] + [P] * 9),
            "gdr_chunk_fwd_fused_prep_workspace_size": (i64, [i64, i64, i64, i32, i32]),
            "gdr_chunk_fwd_fused_prep": (i32, [i64, i64, i64, i32, i32, i32] + [P] * 11 + [i64, P]),
            "gdr_gdp_chunk_fwd_workspace_size": (i64, [i64, i64, i64, i32, i32, i32]),
            "gdr_gdp_chunk_fwd": (i32, [i64, i64, i64, i32, i32, i32, i32] + [P] * 9 + [i64, P]),
            "gdr_gdn2_chunk_fwd_workspace_size": (i64, [i64, i64, i64, i32, i32]),
            "gdr_gdn2_chunk_fwd": (i32, [i64, i64, i64, i32, i32, i32] + [P] * 10 + [i64, P]),
            "gdr_frame_fwd_workspace_size": (i64, [i64, i64, i64, i32, i32, i32]),
            "gdr_frame_fwd": (i32, [i64, i64, i64, i32, i32, i32, i32, i32] + [P] * 9 + [i64, P]),
            "gdr_decode_step": (i32, [i64, i64, i32, i32, i32, i32] + [P] * 8),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def version() -> int:
    return int(load_library().gdr_version())


def status_string(status: int) -> str:
    return load_library().gdr_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which allocations belong to the call's stream (torch's current one if None)."""
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _launch(dev, fn, *args):
    """fn(*args) with the tensors' device current: the library resolves its per-device launch
    settings (and gdr_chunk_fwd_noalloc's built-in workspace) through the current device."""
    import torch
    with torch.cuda.device(dev):
        return fn(*args)


def _io_dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"q/k/v/o must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, shape, dtype, device):
    if t.shape != shape:
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _size(n, where):
    n = int(n)
    if n < 0:
        raise GdrError(GDR_ERR_SHAPE, where)
    return n


def _outputs(o_shape, io_torch_dtype, S_shape, dev, out, final_state, output_final_state, stream):
    import torch
    with _on(stream):
        o = torch.empty(o_shape, dtype=io_torch_dtype, device=dev) if out is None else out
        if output_final_state and final_state is None:
            final_state = torch.empty(S_shape, dtype=torch.float32, device=dev)
    _check(o, "out", o_shape, io_torch_dtype, dev)
    if final_state is not None:
        _check(final_state, "final_state", S_shape, torch.float32, dev)
    return o, final_state


def _workspace(workspace, need, dev, stream):
    """The caller's uint8 workspace tensor, or (None) one allocated on the call's stream."""
    import torch
    if workspace is None:
        if need == 0:
            return None, 0
        with _on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on the inputs' device")
    return workspace, workspace.numel() * workspace.element_size()


def chunk_fwd_workspace_size(B, H, T, d_k, d_v, io_dtype=GDR_BF16, gate=GDR_GATE_SCALAR) -> int:
    """gdr_chunk_fwd_workspace_size: bytes of workspace gdr_chunk_fwd needs (0: none)."""
    return _size(load_library().gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, io_dtype, gate),
                 "gdr_chunk_fwd_workspace_size")


def chunk_fwd(q, k, v, g, beta, initial_state=None, *, output_final_state=True, out=None,
              final_state=None, stream=None, workspace=None):
    """gdr_chunk_fwd on torch tensors.

    q, k [B,H,T,d_k]; v [B,H,T,d_v] (bf16 or fp32); g [B,H,T] or [B,H,T,d_k] fp32
    (log-decay); beta [B,H,T] fp32; initial_state [B,H,d_v,d_k] fp32 or None.
    workspace: a uint8 CUDA tensor of at least chunk_fwd_workspace_size(...) bytes, or None
    (allocated with torch on the call's stream).
    Returns (o, final_state); final_state is None when output_final_state is False.
    """
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd needs GPU tensors")
    io = _io_dtype(q)
    _check(q, "q", (B, H, T, dk), q.dtype, dev)
    _check(k, "k", (B, H, T, dk), q.dtype, dev)
    _check(v, "v", (B, H, T, dv), q.dtype, dev)
    if g.shape == (B, H, T):
        gate = GDR_GATE_SCALAR
    elif g.shape == (B, H, T, dk):
        gate = GDR_GATE_CHANNEL
    else:
        raise ValueError(f"g: expected [B,H,T] or [B,H,T,d_k], got {tuple(g.shape)}")
    _check(g, "g", tuple(g.shape), torch.float32, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, dv, dk), torch.float32, dev)
    o, final_state = _outputs((B, H, T, dv), q.dtype, (B, H, dv, dk), dev, out, final_state, output_final_state,
                              stream)
    need = chunk_fwd_workspace_size(B, H, T, dk, dv, io, gate)
    ws, nbytes = _workspace(workspace, need, dev, stream)
    st = _launch(dev, load_library().gdr_chunk_fwd, B, H, T, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(ws), nbytes,
                                      _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_chunk_fwd")
    return o, final_state


# the size of gdr_chunk_fwd_noalloc's built-in workspace (GDR_CHUNK_FWD_NOALLOC_WORKSPACE_BYTES)
NOALLOC_WORKSPACE_BYTES = 96 << 20


def chunk_fwd_noalloc(q, k, v, g, beta, initial_state, out, final_state, *, stream=None):
    """gdr_chunk_fwd_noalloc on torch tensors: chunk_fwd with the library's built-in workspace.

    Same tensors as chunk_fwd; the outputs ``out`` and ``final_state`` (or None to skip the
    state) are the caller's, so the call allocates nothing.  Raises GdrError with
    GDR_ERR_WORKSPACE when the configuration needs more than NOALLOC_WORKSPACE_BYTES.  Calls on
    one GPU share the built-in workspace: overlapping calls (other streams or threads) race.
    """
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd_noalloc needs GPU tensors")
    io = _io_dtype(q)
    _check(q, "q", (B, H, T, dk), q.dtype, dev)
    _check(k, "k", (B, H, T, dk), q.dtype, dev)
    _check(v, "v", (B, H, T, dv), q.dtype, dev)
    if g.shape == (B, H, T):
        gate = GDR_GATE_SCALAR
    elif g.shape == (B, H, T, dk):
        gate = GDR_GATE_CHANNEL
    else:
        raise ValueError(f"g: expected [B,H,T] or [B,H,T,d_k], got {tuple(g.shape)}")
    _check(g, "g", tuple(g.shape), torch.float32, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, dv, dk), torch.float32, dev)
    _check(out, "out", (B, H, T, dv), q.dtype, dev)
    if final_state is not None:
        _check(final_state, "final_state", (B, H, dv, dk), torch.float32, dev)
    st = _launch(dev, load_library().gdr_chunk_fwd_noalloc, B, H, T, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                              _ptr(beta), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                              _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_chunk_fwd_noalloc")
    return out, final_state


def chunk_fwd_fused_prep_workspace_size(B, H, T, d_k, d_v) -> int:
    return _size(load_library().gdr_chunk_fwd_fused_prep_workspace_size(B, H, T, d_k, d_v),
                 "gdr_chunk_fwd_fused_prep_workspace_size")


def chunk_fwd_fused_prep(q_raw, k_raw, v, dt, A_log, dt_bias, beta_logit, initial_state=None, *,
                         output_final_state=True, out=None, final_state=None, stream=None, workspace=None):
    """gdr_chunk_fwd_fused_prep: the scalar-gate chunked forward from raw projections (q, k
    normalised, beta = sigmoid(beta_logit), g = -exp(A_log) softplus(dt + dt_bias) inside the
    kernels).

    q_raw, k_raw [B,H,T,d_k], v [B,H,T,d_v] (bf16); dt, beta_logit [B,H,T] fp32;
    A_log, dt_bias [H] fp32; initial_state [B,H,d_v,d_k] fp32 or None; workspace as chunk_fwd.
    Returns (o, final_state); final_state is None when output_final_state is False.
    """
    import torch
    B, H, T, dk = q_raw.shape
    dv = v.shape[-1]
    dev = q_raw.device
    if dev.type != "cuda":
        raise ValueError("chunk_fwd_fused_prep needs GPU tensors")
    io = _io_dtype(q_raw)
    _check(k_raw, "k_raw", (B, H, T, dk), q_raw.dtype, dev)
    _check(q_raw, "q_raw", (B, H, T, dk), q_raw.dtype, dev)
    _check(v, "v", (B, H, T, dv), q_raw.dtype, dev)
    _check(dt, "dt", (B, H, T), torch.float32, dev)
    _check(beta_logit, "beta_logit", (B, H, T), torch.float32, dev)
    _check(A_log, "A_log", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, dv, dk), torch.float32, dev)
    o, final_state = _outputs((B, H, T, dv), q_raw.dtype, (B, H, dv, dk), dev, out, final_state,
                              output_final_state, stream)
    ws, nbytes = _workspace(workspace, chunk_fwd_fused_prep_workspace_size(B, H, T, dk, dv), dev, stream)
    st = _launch(dev, load_library().gdr_chunk_fwd_fused_prep, B, H, T, dk, dv, io, _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(dt),
                                                 _ptr(A_log), _ptr(dt_bias), _ptr(beta_logit), _ptr(initial_state),
                                                 _ptr(o), _ptr(final_state), _ptr(ws), nbytes, _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_chunk_fwd_fused_prep")
    return o, final_state


def gdp_chunk_fwd_workspace_size(B, H, T, n_h, d_k, d_v) -> int:
    return _size(load_library().gdr_gdp_chunk_fwd_workspace_size(B, H, T, n_h, d_k, d_v),
                 "gdr_gdp_chunk_fwd_workspace_size")


def gdp_chunk_fwd(q, k, v, g, beta, initial_state=None, *, output_final_state=True, out=None,
                  final_state=None, stream=None, workspace=None):
    """gdr_gdp_chunk_fwd (Gated Delta Product) on torch tensors.

    q [B,H,T,d_k]; k [B,H,T,n_h,d_k]; v [B,H,T,n_h,d_v] (bf16); g [B,H,T] fp32 (one
    log-decay per token); beta [B,H,T,n_h] fp32; initial_state [B,H,d_v,d_k] fp32 or None;
    workspace as chunk_fwd.
    Returns (o [B,H,T,d_v], final_state); final_state is None when output_final_state is False.
    """
    import torch
    B, H, T, dk = q.shape
    if k.dim() != 5:
        raise ValueError(f"k: expected [B,H,T,n_h,d_k], got {tuple(k.shape)}")
    nh = k.shape[3]
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdp_chunk_fwd needs GPU tensors")
    io = _io_dtype(q)
    _check(q, "q", (B, H, T, dk), q.dtype, dev)
    _check(k, "k", (B, H, T, nh, dk), q.dtype, dev)
    _check(v, "v", (B, H, T, nh, dv), q.dtype, dev)
    _check(g, "g", (B, H, T), torch.float32, dev)
    _check(beta, "beta", (B, H, T, nh), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, dv, dk), torch.float32, dev)
    o, final_state = _outputs((B, H, T, dv), q.dtype, (B, H, dv, dk), dev, out, final_state, output_final_state,
                              stream)
    ws, nbytes = _workspace(workspace, gdp_chunk_fwd_workspace_size(B, H, T, nh, dk, dv), dev, stream)
    st = _launch(dev, load_library().gdr_gdp_chunk_fwd, B, H, T, nh, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(ws), nbytes,
                                          _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_gdp_chunk_fwd")
    return o, final_state


def gdn2_chunk_fwd_workspace_size(B, H, T, d_k, d_v) -> int:
    return _size(load_library().gdr_gdn2_chunk_fwd_workspace_size(B, H, T, d_k, d_v),
                 "gdr_gdn2_chunk_fwd_workspace_size")


def gdn2_chunk_fwd(q, k, v, g, b, w, initial_state=None, *, output_final_state=True, out=None,
                   final_state=None, stream=None, workspace=None):
    """gdr_gdn2_chunk_fwd (Gated DeltaNet-2) on torch tensors.

    q, k [B,H,T,d_k]; v [B,H,T,d_v] (bf16); g [B,H,T,d_k] fp32 (per-channel log-decay);
    b [B,H,T,d_k] fp32 (erase gate); w [B,H,T,d_v] fp32 (write gate); initial_state
    [B,H,d_v,d_k] fp32 or None; workspace as chunk_fwd.
    Returns (o, final_state); final_state is None when output_final_state is False.
    """
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("gdn2_chunk_fwd needs GPU tensors")
    io = _io_dtype(q)
    _check(q, "q", (B, H, T, dk), q.dtype, dev)
    _check(k, "k", (B, H, T, dk), q.dtype, dev)
    _check(v, "v", (B, H, T, dv), q.dtype, dev)
    _check(g, "g", (B, H, T, dk), torch.float32, dev)
    _check(b, "b", (B, H, T, dk), torch.float32, dev)
    _check(w, "w", (B, H, T, dv), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, dv, dk), torch.float32, dev)
    o, final_state = _outputs((B, H, T, dv), q.dtype, (B, H, dv, dk), dev, out, final_state, output_final_state,
                              stream)
    ws, nbytes = _workspace(workspace, gdn2_chunk_fwd_workspace_size(B, H, T, dk, dv), dev, stream)
    st = _launch(dev, load_library().gdr_gdn2_chunk_fwd, B, H, T, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                                           _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(ws), nbytes,
                                           _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_gdn2_chunk_fwd")
    return o, final_state


def frame_fwd_workspace_size(B, H, T, frame_len, d_k, d_v) -> int:
    return _size(load_library().gdr_frame_fwd_workspace_size(B, H, T, frame_len, d_k, d_v),
                 "gdr_frame_fwd_workspace_size")


def frame_fwd(q, k, v, gamma, g, frame_len, initial_state=None, *, output_final_state=True, out=None,
              final_state=None, workspace=None, stream=None):
    """gdr_frame_fwd (frame-level implicit update) on torch tensors.

    q, k [B,H,T,d_k]; v [B,H,T,d_v] (bf16); gamma [B,H,T] fp32; g [B,H,F] or [B,H,F,d_k]
    fp32 (log forget gate per frame, F = ceil(T / frame_len)); initial_state [B,H,d_v,d_k]
    fp32 or None; workspace as chunk_fwd.
    Returns (o, final_state); final_state is None when output_final_state is False.
    """
    import torch
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("frame_fwd needs GPU tensors")
    io = _io_dtype(q)
    F = (T + frame_len - 1) // frame_len
    _check(k, "k", (B, H, T, dk), q.dtype, dev)
    _check(v, "v", (B, H, T, dv), q.dtype, dev)
    _check(gamma, "gamma", (B, H, T), torch.float32, dev)
    if g.shape == (B, H, F):
        gate = GDR_GATE_SCALAR
    elif g.shape == (B, H, F, dk):
        gate = GDR_GATE_CHANNEL
    else:
        raise ValueError(f"g: expected [B,H,F] or [B,H,F,d_k] with F={F}, got {tuple(g.shape)}")
    _check(g, "g", tuple(g.shape), torch.float32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, dv, dk), torch.float32, dev)
    o, final_state = _outputs((B, H, T, dv), q.dtype, (B, H, dv, dk), dev, out, final_state, output_final_state,
                              stream)
    ws, nbytes = _workspace(workspace, frame_fwd_workspace_size(B, H, T, frame_len, dk, dv), dev, stream)
    st = _launch(dev, load_library().gdr_frame_fwd, B, H, T, frame_len, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                      _ptr(g), _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(ws), nbytes,
                                      _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_frame_fwd")
    return o, final_state


def decode_step(q, k, v, g, beta, state, *, out=None, stream=None):
    """gdr_decode_step on torch tensors; ``state`` [N,H,d_v,d_k] fp32 is updated in place.

    q, k [N,H,d_k]; v [N,H,d_v] (bf16 or fp32); g [N,H] or [N,H,d_k] fp32; beta [N,H] fp32.
    Returns o [N,H,d_v]."""
    import torch
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_step needs GPU tensors")
    io = _io_dtype(q)
    _check(k, "k", (N, H, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    if g.shape == (N, H):
        gate = GDR_GATE_SCALAR
    elif g.shape == (N, H, dk):
        gate = GDR_GATE_CHANNEL
    else:
        raise ValueError(f"g: expected [N,H] or [N,H,d_k], got {tuple(g.shape)}")
    _check(g, "g", tuple(g.shape), torch.float32, dev)
    _check(beta, "beta", (N, H), torch.float32, dev)
    _check(state, "state", (N, H, dv, dk), torch.float32, dev)
    with _on(stream):
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", (N, H, dv), q.dtype, dev)
    st = _launch(dev, load_library().gdr_decode_step, N, H, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(state), _ptr(o), _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_decode_step")
    return o
