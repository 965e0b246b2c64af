"""ctypes binding of libgdr (include/gdr.h): argument marshalling only.

PyTorch provides device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libgdr.so")

GDR_OK = 0
GDR_ERR_SHAPE = 2
GDR_BF16, GDR_F32 = 0, 1
GDR_GATE_SCALAR, GDR_GATE_CHANNEL = 0, 1

# every entry point include/gdr.h declares
EXPORTED_SYMBOLS = ("gdr_version", "gdr_status_string", "gdr_chunk_fwd", "gdr_chunk_fwd_workspace_size",
                    "gdr_chunk_fwd_ws", "gdr_chunk_fwd_fused_prep",
                    "gdr_chunk_fwd_fused_prep_workspace_size", "gdr_chunk_fwd_fused_prep_ws", "gdr_gdp_chunk_fwd", "gdr_gdp_chunk_fwd_workspace_size", "gdr_gdp_chunk_fwd_ws", "gdr_gdn2_chunk_fwd",
                    "gdr_gdn2_chunk_fwd_workspace_size", "gdr_gdn2_chunk_fwd_ws", "gdr_frame_fwd_workspace_size", "gdr_frame_fwd", "gdr_decode_step")

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
        lib.gdr_version.restype = i32
        lib.gdr_version.argtypes = []
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_status_string.argtypes = [i32]
        lib.gdr_chunk_fwd.restype = i32
        lib.gdr_chunk_fwd.argtypes = [i64, i64, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]
        lib.gdr_chunk_fwd_workspace_size.restype = i64
        lib.gdr_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, i32]
        lib.gdr_chunk_fwd_ws.restype = i32
        lib.gdr_chunk_fwd_ws.argtypes = [i64, i64, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, i64, P]
        lib.gdr_chunk_fwd_fused_prep.restype = i32
        lib.gdr_chunk_fwd_fused_prep.argtypes = [i64, i64, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P]
        lib.gdr_chunk_fwd_fused_prep_workspace_size.restype = i64
        lib.gdr_chunk_fwd_fused_prep_workspace_size.argtypes = [i64, i64, i64, i32, i32]
        lib.gdr_chunk_fwd_fused_prep_ws.restype = i32
        lib.gdr_chunk_fwd_fused_prep_ws.argtypes = [i64, i64, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P,
                                                    i64, P]
        lib.gdr_gdp_chunk_fwd.restype = i32
        lib.gdr_gdp_chunk_fwd.argtypes = [i64, i64, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]
        lib.gdr_gdp_chunk_fwd_workspace_size.restype = i64
        lib.gdr_gdp_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32]
        lib.gdr_gdp_chunk_fwd_ws.restype = i32
        lib.gdr_gdp_chunk_fwd_ws.argtypes = [i64, i64, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, i64, P]
        lib.gdr_gdn2_chunk_fwd.restype = i32
        lib.gdr_gdn2_chunk_fwd.argtypes = [i64, i64, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
        lib.gdr_gdn2_chunk_fwd_workspace_size.restype = i64
        lib.gdr_gdn2_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i32, i32]
        lib.gdr_gdn2_chunk_fwd_ws.restype = i32
        lib.gdr_gdn2_chunk_fwd_ws.argtypes = [i64, i64, i64, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, i64, P]
        lib.gdr_frame_fwd_workspace_size.restype = i64
        lib.gdr_frame_fwd_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32]
        lib.gdr_frame_fwd.restype = i32
        lib.gdr_frame_fwd.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, i64, P]
        lib.gdr_decode_step.restype = i32
        lib.gdr_decode_step.argtypes = [i64, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
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


def chunk_fwd_workspace_size(B, H, T, d_k, d_v, io_dtype=GDR_BF16, gate=GDR_GATE_SCALAR) -> int:
    """gdr_chunk_fwd_workspace_size: bytes of workspace the two-kernel path needs (0: none)."""
    n = int(load_library().gdr_chunk_fwd_workspace_size(B, H, T, d_k, d_v, io_dtype, gate))
    if n < 0:
        raise GdrError(GDR_ERR_SHAPE, "gdr_chunk_fwd_workspace_size")
    return n


def chunk_fwd(q, k, v, g, beta, initial_state=None, *, output_final_state=True, out=None,
              final_state=None, stream=None, workspace="auto"):
    """The chunked forward on torch tensors.

    q, k [B,H,T,d_k]; v [B,H,T,d_v] (bf16 or fp32); g [B,H,T] or [B,H,T,d_k] fp32
    (log-decay); beta [B,H,T] fp32; initial_state [B,H,d_v,d_k] fp32 or None.
    workspace: "auto" (default) allocates the two-kernel path's workspace with torch and
    calls gdr_chunk_fwd_ws; a uint8 CUDA tensor is used as that workspace; None calls
    gdr_chunk_fwd (one kernel, no workspace).
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
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", (B, H, T, dv), q.dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (B, H, dv, dk), torch.float32, dev)
    if workspace is None:
        st = load_library().gdr_chunk_fwd(B, H, T, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                          _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                          _stream(stream, dev))
        if st != GDR_OK:
            raise GdrError(st, "gdr_chunk_fwd")
        return o, final_state
    need = chunk_fwd_workspace_size(B, H, T, dk, dv, io, gate)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace: expected 'auto', None or a tensor, got {workspace!r}")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on the inputs' device")
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().gdr_chunk_fwd_ws(B, H, T, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(workspace), nbytes,
                                         _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_chunk_fwd_ws")
    return o, final_state


def chunk_fwd_fused_prep_workspace_size(B, H, T, d_k, d_v) -> int:
    n = int(load_library().gdr_chunk_fwd_fused_prep_workspace_size(B, H, T, d_k, d_v))
    if n < 0:
        raise GdrError(GDR_ERR_SHAPE, "gdr_chunk_fwd_fused_prep_workspace_size")
    return n


def chunk_fwd_fused_prep(q_raw, k_raw, v, dt, A_log, dt_bias, beta_logit, initial_state=None, *,
                         output_final_state=True, out=None, final_state=None, stream=None, workspace="auto"):
    """The scalar-gate chunked forward from raw projections (q, k normalised, beta =
    sigmoid(beta_logit), g = -exp(A_log) softplus(dt + dt_bias) inside the kernels):
    gdr_chunk_fwd_fused_prep_ws, or gdr_chunk_fwd_fused_prep with workspace=None.

    q_raw, k_raw [B,H,T,d_k], v [B,H,T,d_v] (bf16); dt, beta_logit [B,H,T] fp32;
    A_log, dt_bias [H] fp32; initial_state [B,H,d_v,d_k] fp32 or None.  workspace: "auto"
    (default) allocates the two-kernel path's workspace with torch; a uint8 CUDA tensor is used
    as that workspace; None calls the single kernel.
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
    o = torch.empty((B, H, T, dv), dtype=q_raw.dtype, device=dev) if out is None else out
    _check(o, "out", (B, H, T, dv), q_raw.dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (B, H, dv, dk), torch.float32, dev)
    if workspace is None:
        st = load_library().gdr_chunk_fwd_fused_prep(B, H, T, dk, dv, io, _ptr(q_raw), _ptr(k_raw), _ptr(v),
                                                     _ptr(dt), _ptr(A_log), _ptr(dt_bias), _ptr(beta_logit),
                                                     _ptr(initial_state), _ptr(o), _ptr(final_state),
                                                     _stream(stream, dev))
        if st != GDR_OK:
            raise GdrError(st, "gdr_chunk_fwd_fused_prep")
        return o, final_state
    need = chunk_fwd_fused_prep_workspace_size(B, H, T, dk, dv)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace: expected 'auto', None or a tensor, got {workspace!r}")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on the inputs' device")
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().gdr_chunk_fwd_fused_prep_ws(B, H, T, dk, dv, io, _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(dt),
                                                    _ptr(A_log), _ptr(dt_bias), _ptr(beta_logit),
                                                    _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(workspace),
                                                    nbytes, _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_chunk_fwd_fused_prep_ws")
    return o, final_state


def gdp_chunk_fwd_workspace_size(B, H, T, n_h, d_k, d_v) -> int:
    n = int(load_library().gdr_gdp_chunk_fwd_workspace_size(B, H, T, n_h, d_k, d_v))
    if n < 0:
        raise GdrError(GDR_ERR_SHAPE, "gdr_gdp_chunk_fwd_workspace_size")
    return n


def gdp_chunk_fwd(q, k, v, g, beta, initial_state=None, *, output_final_state=True, out=None,
                  final_state=None, stream=None, workspace="auto"):
    """Gated Delta Product (gdr_gdp_chunk_fwd_ws, or gdr_gdp_chunk_fwd) on torch tensors.

    q [B,H,T,d_k]; k [B,H,T,n_h,d_k]; v [B,H,T,n_h,d_v] (bf16); g [B,H,T] fp32 (one
    log-decay per token); beta [B,H,T,n_h] fp32; initial_state [B,H,d_v,d_k] fp32 or None.
    workspace: "auto" (default) allocates the two-kernel path's workspace with torch; a uint8
    CUDA tensor is used as that workspace; None calls the single kernel.
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
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", (B, H, T, dv), q.dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (B, H, dv, dk), torch.float32, dev)
    if workspace is None:
        st = load_library().gdr_gdp_chunk_fwd(B, H, T, nh, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                              _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                              _stream(stream, dev))
        if st != GDR_OK:
            raise GdrError(st, "gdr_gdp_chunk_fwd")
        return o, final_state
    need = gdp_chunk_fwd_workspace_size(B, H, T, nh, dk, dv)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace: expected 'auto', None or a tensor, got {workspace!r}")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on the inputs' device")
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().gdr_gdp_chunk_fwd_ws(B, H, T, nh, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                             _ptr(beta), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                             _ptr(workspace), nbytes, _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_gdp_chunk_fwd_ws")
    return o, final_state


def gdn2_chunk_fwd_workspace_size(B, H, T, d_k, d_v) -> int:
    n = int(load_library().gdr_gdn2_chunk_fwd_workspace_size(B, H, T, d_k, d_v))
    if n < 0:
        raise GdrError(GDR_ERR_SHAPE, "gdr_gdn2_chunk_fwd_workspace_size")
    return n


def gdn2_chunk_fwd(q, k, v, g, b, w, initial_state=None, *, output_final_state=True, out=None,
                   final_state=None, stream=None, workspace="auto"):
    """Gated DeltaNet-2 (gdr_gdn2_chunk_fwd_ws, or gdr_gdn2_chunk_fwd) on torch tensors.

    q, k [B,H,T,d_k]; v [B,H,T,d_v] (bf16); g [B,H,T,d_k] fp32 (per-channel log-decay);
    b [B,H,T,d_k] fp32 (erase gate); w [B,H,T,d_v] fp32 (write gate); initial_state
    [B,H,d_v,d_k] fp32 or None.  workspace: "auto" (default) allocates the two-kernel path's
    workspace with torch; a uint8 CUDA tensor is used as that workspace; None calls the
    single kernel.  Returns (o, final_state); final_state is None when output_final_state is
    False.
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
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", (B, H, T, dv), q.dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (B, H, dv, dk), torch.float32, dev)
    if workspace is None:
        st = load_library().gdr_gdn2_chunk_fwd(B, H, T, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b),
                                               _ptr(w), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                               _stream(stream, dev))
        if st != GDR_OK:
            raise GdrError(st, "gdr_gdn2_chunk_fwd")
        return o, final_state
    need = gdn2_chunk_fwd_workspace_size(B, H, T, dk, dv)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace: expected 'auto', None or a tensor, got {workspace!r}")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous tensor on the inputs' device")
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().gdr_gdn2_chunk_fwd_ws(B, H, T, dk, dv, io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b),
                                              _ptr(w), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                              _ptr(workspace), nbytes, _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_gdn2_chunk_fwd_ws")
    return o, final_state


def frame_fwd_workspace_size(B, H, T, frame_len, d_k, d_v) -> int:
    n = int(load_library().gdr_frame_fwd_workspace_size(B, H, T, frame_len, d_k, d_v))
    if n < 0:
        raise GdrError(GDR_ERR_SHAPE, "gdr_frame_fwd_workspace_size")
    return n


def frame_fwd(q, k, v, gamma, g, frame_len, initial_state=None, *, output_final_state=True, out=None,
              final_state=None, workspace=None, stream=None):
    """gdr_frame_fwd (frame-level implicit update) on torch tensors.

    q, k [B,H,T,d_k]; v [B,H,T,d_v] (bf16); gamma [B,H,T] fp32; g [B,H,F] or [B,H,F,d_k]
    fp32 (log forget gate per frame, F = ceil(T / frame_len)); initial_state [B,H,d_v,d_k]
    fp32 or None; workspace: a uint8 CUDA tensor or None (allocated with torch).
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
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", (B, H, T, dv), q.dtype, dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (B, H, dv, dk), torch.float32, dev)
    if workspace is None:
        workspace = torch.empty(max(frame_fwd_workspace_size(B, H, T, frame_len, dk, dv), 1), dtype=torch.uint8,
                                device=dev)
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().gdr_frame_fwd(B, H, T, frame_len, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(gamma),
                                      _ptr(g), _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(workspace),
                                      nbytes, _stream(stream, dev))
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
    o = torch.empty((N, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", (N, H, dv), q.dtype, dev)
    st = load_library().gdr_decode_step(N, H, dk, dv, io, gate, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(state), _ptr(o), _stream(stream, dev))
    if st != GDR_OK:
        raise GdrError(st, "gdr_decode_step")
    return o
