"""C-ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects invalid arguments on the host before enqueuing
anything (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_15_amd as gdr
from gated_delta_rule_15_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

OK, INVALID, SHAPE, DTYPE, UNSUP, WSERR, HIPERR = 0, 1, 2, 3, 4, 5, 6
FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every call below fails validation
FAKE2 = ctypes.c_void_p(0x20000000)
WS = ctypes.c_void_p(0x50000000)      # a fake workspace that overlaps no other fake buffer


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdr.LIBRARY_PATH):
        pytest.skip("libgdr.so is not built")
    return gdr.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(B.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {gdr.LIBRARY_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_version_and_status_strings(lib):
    assert gdr.version() == 200
    for s in range(7):
        assert gdr.status_string(s) and "unknown" not in gdr.status_string(s)
    assert "workspace" in gdr.status_string(WSERR)
    assert "unknown" in gdr.status_string(99)


def chunk(lib, B=1, H=1, T=64, dk=128, dv=128, io=0, gate=0, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
          s0=None, o=FAKE2, sf=None, ws=WS, nbytes=1 << 20):
    return lib.gdr_chunk_fwd(B, H, T, dk, dv, io, gate, q, k, v, g, beta, s0, o, sf, ws, nbytes, None)


def decode(lib, N=1, H=1, dk=128, dv=128, io=0, gate=0, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S=FAKE2,
           o=ctypes.c_void_p(0x40000000)):
    return lib.gdr_decode_step(N, H, dk, dv, io, gate, q, k, v, g, beta, S, o, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(H=-2), INVALID), (dict(T=-1), INVALID),
    (dict(dk=96), SHAPE), (dict(dk=256), SHAPE), (dict(dv=48), SHAPE), (dict(dv=0), SHAPE), (dict(dv=288), SHAPE),
    (dict(io=2), DTYPE), (dict(gate=5), INVALID),
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(g=None), INVALID),
    (dict(beta=None), INVALID), (dict(o=None), INVALID),
    (dict(o=FAKE), INVALID),                                   # o overlaps q
    (dict(io=1, dk=128), UNSUP),                               # fp32 chunk path is d_k = 64 only
    (dict(io=1, dk=64, dv=64, gate=1), UNSUP),                 # per-channel gate needs bf16 I/O
    (dict(B=1 << 40, H=1 << 30), SHAPE),                       # size overflow
    (dict(T=(1 << 22) + 1), SHAPE),                            # 32-bit per-sequence offsets
    (dict(ws=None), WSERR),                                    # a workspace is required
    (dict(nbytes=12863), WSERR),                               # one chunk needs 12864 bytes
    (dict(nbytes=-1), WSERR),
    (dict(ws=FAKE), WSERR),                                    # workspace overlaps q
    (dict(ws=FAKE2), WSERR),                                   # workspace overlaps o
    (dict(gate=1, nbytes=61951), WSERR),                       # channel gate: 61952 bytes per chunk
])
def test_chunk_fwd_rejects(lib, kw, status):
    assert chunk(lib, **kw) == status


def test_chunk_fwd_state_aliasing_rules(lib):
    s = ctypes.c_void_p(0x30000000)
    s_shift = ctypes.c_void_p(0x30000000 + 4)
    # partial overlap of initial and final state is rejected (exact aliasing is allowed,
    # checked on the GPU)
    assert chunk(lib, s0=s, sf=s_shift) == INVALID


def test_chunk_fwd_empty_batch_is_a_noop(lib):
    assert chunk(lib, B=0) == OK
    assert chunk(lib, H=0, q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, nbytes=0) == OK
    assert chunk(lib, T=0, q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, nbytes=0) == OK


def test_chunk_fwd_f32_needs_no_workspace(lib):
    # fp32 I/O queries 0 bytes; the workspace argument is then ignored (validation passes and the
    # call would launch, so only the no-op shape is called here)
    assert lib.gdr_chunk_fwd_workspace_size(1, 1, 64, 64, 64, 1, 0) == 0
    assert chunk(lib, B=0, io=1, dk=64, dv=64, ws=None, nbytes=0) == OK


def noalloc(lib, B=1, H=1, T=64, dk=128, dv=128, io=0, gate=0, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
            s0=None, o=FAKE2, sf=None):
    return lib.gdr_chunk_fwd_noalloc(B, H, T, dk, dv, io, gate, q, k, v, g, beta, s0, o, sf, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(dk=96), SHAPE), (dict(io=2), DTYPE), (dict(q=None), INVALID),
    (dict(o=FAKE), INVALID), (dict(io=1, dk=128), UNSUP), (dict(T=(1 << 22) + 1), SHAPE),
    (dict(B=8, H=16, T=4096), WSERR),                          # 132.5 MiB of records: beyond the 96 MiB built in
    (dict(B=1, H=16, T=8192, gate=1), WSERR),                  # channel gate: 16 x 128 x 61952 bytes
])
def test_chunk_fwd_noalloc_rejects(lib, kw, status):
    assert noalloc(lib, **kw) == status


def test_chunk_fwd_noalloc_limit(lib):
    n = lib.gdr_chunk_fwd_workspace_size
    assert n(4, 16, 4096, 128, 128, 0, 0) <= B.NOALLOC_WORKSPACE_BYTES   # the B=4 H=16 T=4096 shape fits
    assert n(8, 16, 4096, 128, 128, 0, 0) > B.NOALLOC_WORKSPACE_BYTES
    text = open(HEADER).read()
    assert re.search(r"#define GDR_CHUNK_FWD_NOALLOC_WORKSPACE_BYTES \(96u << 20\)", text)
    assert B.NOALLOC_WORKSPACE_BYTES == 96 << 20
    assert noalloc(lib, B=0) == OK and noalloc(lib, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def test_workspace_size(lib):
    n = lib.gdr_chunk_fwd_workspace_size
    assert n(4, 16, 4096, 128, 128, 0, 0) == 64 * 64 * 12864        # A^T, T, factors per (sequence, chunk)
    assert n(1, 1, 65, 64, 32, 0, 0) == 2 * 12864                    # ragged tail counts as a chunk
    assert n(1, 1, 0, 128, 128, 0, 0) == 0
    assert n(2, 2, 100, 64, 64, 1, 0) == 0                           # fp32 I/O: one kernel, no workspace
    assert n(2, 2, 100, 128, 64, 1, 0) == -1                         # fp32 I/O is d_k = 64 only
    assert n(2, 2, 100, 128, 128, 0, 1) == 4 * 2 * 61952             # channel gate: 12288 + 388 d_k
    assert n(1, 3, 64, 64, 64, 0, 1) == 3 * 37120
    assert n(1, 1, 1 << 22, 128, 32, 0, 1) == 65536 * 61952          # longest sequence: below 4 GiB
    assert n(1, 1, 64, 96, 128, 0, 0) == -1 and n(-1, 1, 64, 128, 128, 0, 0) == -1
    assert n(1, 1, (1 << 22) + 1, 128, 128, 0, 0) == -1
    assert gdr.chunk_fwd_workspace_size(1, 2, 128, 128, 128) == 2 * 2 * 12864


def gdp(lib, B=1, H=1, T=64, nh=2, dk=128, dv=128, io=0, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
        s0=None, o=FAKE2, sf=None, ws=WS, nbytes=1 << 20):
    return lib.gdr_gdp_chunk_fwd(B, H, T, nh, dk, dv, io, q, k, v, g, beta, s0, o, sf, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(T=-1), INVALID), (dict(nh=0), INVALID), (dict(nh=-3), INVALID),
    (dict(nh=17), SHAPE), (dict(dk=96), SHAPE), (dict(dv=16), SHAPE), (dict(io=7), DTYPE),
    (dict(io=1), UNSUP),                                        # bf16 I/O only
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(g=None), INVALID),
    (dict(beta=None), INVALID), (dict(o=None), INVALID),
    (dict(o=FAKE), INVALID),                                    # o overlaps q
    (dict(T=1 << 21, nh=3), SHAPE),                             # T * n_h above 2^22
    (dict(T=(1 << 22) + 1, nh=1), SHAPE),
    (dict(B=1 << 40, H=1 << 30), SHAPE),                        # size overflow
    (dict(ws=None), WSERR),                                     # a workspace is required
    (dict(nbytes=2 * 12864 - 1), WSERR),                        # 128 virtual steps: two records
    (dict(nbytes=-1), WSERR),
    (dict(ws=FAKE), WSERR), (dict(ws=FAKE2), WSERR),            # workspace overlaps q / o
])
def test_gdp_chunk_fwd_rejects(lib, kw, status):
    assert gdp(lib, **kw) == status


def test_gdp_chunk_fwd_empty_batch_is_a_noop(lib):
    assert gdp(lib, B=0) == OK
    assert gdp(lib, H=0, q=None, k=None, v=None, g=None, beta=None, o=None, ws=None, nbytes=0) == OK


def test_gdp_workspace_size(lib):
    n = lib.gdr_gdp_chunk_fwd_workspace_size
    assert n(4, 16, 2048, 2, 128, 128) == 64 * 64 * 12864
    assert n(1, 1, 33, 2, 64, 64) == 2 * 12864                      # 66 virtual steps: two chunks
    assert n(1, 1, 0, 2, 128, 128) == 0
    assert n(1, 1, 64, 0, 128, 128) == -1 and n(1, 1, 64, 17, 128, 128) == -1


def test_gdp_partial_state_overlap_rejected(lib):
    s = ctypes.c_void_p(0x30000000)
    assert gdp(lib, s0=s, sf=ctypes.c_void_p(0x30000000 + 4)) == INVALID


def gdn2(lib, B=1, H=1, T=64, dk=128, dv=128, io=0, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, w=FAKE,
         s0=None, o=FAKE2, sf=None, ws=WS, nbytes=1 << 20):
    return lib.gdr_gdn2_chunk_fwd(B, H, T, dk, dv, io, q, k, v, g, b, w, s0, o, sf, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(T=-1), INVALID), (dict(dk=96), SHAPE), (dict(dv=48), SHAPE),
    (dict(io=5), DTYPE), (dict(io=1), UNSUP),
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(g=None), INVALID),
    (dict(b=None), INVALID), (dict(w=None), INVALID), (dict(o=None), INVALID),
    (dict(o=FAKE), INVALID),                                    # o overlaps q
    (dict(T=(1 << 22) + 1), SHAPE),
    (dict(T=1 << 22, dv=256), SHAPE),                           # fp32 write gate past 32-bit offsets
    (dict(B=1 << 40, H=1 << 30), SHAPE),
    (dict(ws=None), WSERR),                                     # a workspace is required
    (dict(nbytes=61951), WSERR),                                # one chunk needs 61952 bytes
    (dict(nbytes=-1), WSERR),
    (dict(ws=FAKE), WSERR), (dict(ws=FAKE2), WSERR),            # workspace overlaps q / o
])
def test_gdn2_chunk_fwd_rejects(lib, kw, status):
    assert gdn2(lib, **kw) == status


def test_gdn2_chunk_fwd_empty_batch_is_a_noop(lib):
    assert gdn2(lib, B=0) == OK
    assert gdn2(lib, H=0, q=None, k=None, v=None, g=None, b=None, w=None, o=None, ws=None, nbytes=0) == OK


def test_gdn2_workspace_size(lib):
    n = lib.gdr_gdn2_chunk_fwd_workspace_size
    assert n(2, 2, 100, 128, 128) == 4 * 2 * 61952
    assert n(1, 3, 64, 64, 64) == 3 * 37120
    assert n(1, 1, 0, 128, 128) == 0
    assert n(-1, 1, 64, 128, 128) == -1 and n(1, 1, 64, 96, 128) == -1
    assert n(1, 1, 1 << 22, 128, 32) == 65536 * 61952                # longest sequence: below 4 GiB


def prep(lib, B=1, H=1, T=64, dk=128, dv=128, io=0, q=FAKE, k=FAKE, v=FAKE, dt=FAKE, A=FAKE, bias=FAKE,
         bl=FAKE, s0=None, o=FAKE2, sf=None, ws=WS, nbytes=1 << 20):
    return lib.gdr_chunk_fwd_fused_prep(B, H, T, dk, dv, io, q, k, v, dt, A, bias, bl, s0, o, sf, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(H=-1), INVALID), (dict(T=-1), INVALID), (dict(dk=32), SHAPE),
    (dict(dv=40), SHAPE), (dict(io=3), DTYPE), (dict(io=1), UNSUP),
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(dt=None), INVALID),
    (dict(A=None), INVALID), (dict(bias=None), INVALID), (dict(bl=None), INVALID), (dict(o=None), INVALID),
    (dict(o=FAKE), INVALID),                                    # o overlaps q_raw
    (dict(T=(1 << 22) + 1), SHAPE),
    (dict(B=1 << 40, H=1 << 30), SHAPE),
    (dict(ws=None), WSERR),                                     # a workspace is required
    (dict(nbytes=13119), WSERR),                                # one chunk needs 13120 bytes
    (dict(nbytes=-1), WSERR),
    (dict(ws=FAKE), WSERR), (dict(ws=FAKE2), WSERR),            # workspace overlaps q_raw / o
])
def test_fused_prep_rejects(lib, kw, status):
    assert prep(lib, **kw) == status


def test_fused_prep_workspace_size(lib):
    n = lib.gdr_chunk_fwd_fused_prep_workspace_size
    assert n(4, 16, 4096, 128, 128) == 64 * 64 * 13120
    assert n(1, 2, 65, 64, 64) == 2 * 2 * 13120
    assert n(1, 1, 0, 128, 128) == 0
    assert n(-1, 1, 64, 128, 128) == -1 and n(1, 1, 64, 96, 128) == -1


def test_fused_prep_empty_batch_is_a_noop(lib):
    assert prep(lib, B=0) == OK
    assert prep(lib, T=0, q=None, k=None, v=None, dt=None, bl=None, o=None, ws=None, nbytes=0) == OK


def frame(lib, B=1, H=1, T=64, n=16, dk=128, dv=128, io=0, gate=0, q=FAKE, k=FAKE, v=FAKE, gm=FAKE, g=FAKE,
          s0=None, o=FAKE2, sf=None, w=ctypes.c_void_p(0x50000000), nbytes=1 << 24):
    return lib.gdr_frame_fwd(B, H, T, n, dk, dv, io, gate, q, k, v, gm, g, s0, o, sf, w, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID), (dict(n=0), INVALID), (dict(n=24), SHAPE), (dict(dk=96), SHAPE),
    (dict(dv=32), UNSUP), (dict(dv=256), UNSUP), (dict(io=1, dk=64, dv=64), UNSUP), (dict(io=3), DTYPE),
    (dict(gate=2), INVALID), (dict(q=None), INVALID), (dict(gm=None), INVALID), (dict(g=None), INVALID),
    (dict(o=FAKE), INVALID), (dict(w=None), WSERR), (dict(nbytes=100), WSERR), (dict(w=FAKE), WSERR),
    (dict(nbytes=-1), WSERR),
    (dict(T=(1 << 22) + 1), SHAPE),
    (dict(T=1 << 22, n=16), SHAPE),                             # frames' records past 32-bit offsets
    (dict(T=16 * 131071, n=16, dk=64, dv=128), SHAPE),          # C of one sequence reaches 4 GiB
])
def test_frame_fwd_rejects(lib, kw, status):
    assert frame(lib, **kw) == status


def test_frame_workspace_size(lib):
    n = lib.gdr_frame_fwd_workspace_size
    per = 128 * 128 * 4 + 128 * 128 * 4 + 128 * 128 * 2 + 8 * 4     # W hi+lo, C, S, S's exponents per frame
    assert n(1, 2, 1000, 256, 128, 128) == 2 * 4 * per
    assert n(1, 1, 0, 16, 64, 64) == 0
    assert n(1, 1, 64, 24, 128, 128) == -1 and n(1, 1, 64, 16, 128, 32) == -1
    # one sequence's fp32 C records are addressed with 32-bit offsets (a frame past the end
    # included): d_k = 64, d_v = 128, frame_len = 16 fits up to 131070 frames
    assert n(1, 1, 16 * 131070, 16, 64, 128) > 0
    assert n(1, 1, 16 * 131071, 16, 64, 128) == -1
    assert frame(lib, B=0) == OK


@pytest.mark.parametrize("nh", range(2, 17))
def test_virtual_step_division(nh):
    """The GDP kernel splits virtual step m into (m // n_h, m % n_h) as umulhi(m, ceil(2^32 / n_h)),
    exact for every m below 2^23 (T * n_h <= 2^22 plus a chunk of overhang)."""
    import numpy as np
    magic = np.uint64(((1 << 32) + nh - 1) // nh)
    m = np.arange(1 << 23, dtype=np.uint64)
    assert np.array_equal((m * magic) >> np.uint64(32), m // np.uint64(nh))


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), INVALID), (dict(dk=32), SHAPE), (dict(dv=100), SHAPE), (dict(io=9), DTYPE),
    (dict(gate=2), INVALID), (dict(q=None), INVALID), (dict(S=None), INVALID), (dict(o=None), INVALID),
    (dict(o=FAKE2), INVALID),                                  # o overlaps the state
])
def test_decode_rejects(lib, kw, status):
    assert decode(lib, **kw) == status


def test_decode_empty_is_a_noop(lib):
    assert decode(lib, N=0, q=None, S=None, o=None) == OK


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        gdr.chunk_fwd(x, x, x, torch.zeros(1, 1, 4), torch.zeros(1, 1, 4))
    with pytest.raises(ValueError):
        gdr.gdp_chunk_fwd(x, x[:, :, :, None], x[:, :, :, None], torch.zeros(1, 1, 4), torch.zeros(1, 1, 4, 1))
    with pytest.raises(ValueError):
        gdr.gdn2_chunk_fwd(x, x, x, x, x, x)
    with pytest.raises(ValueError):
        gdr.frame_fwd(x, x, x, torch.zeros(1, 1, 4), torch.zeros(1, 1, 1), 16)
    with pytest.raises(ValueError):
        gdr.chunk_fwd_fused_prep(x, x, x, torch.zeros(1, 1, 4), torch.zeros(1), torch.zeros(1), torch.zeros(1, 1, 4))
    with pytest.raises(ValueError):
        gdr.decode_step(x[:, :, 0], x[:, :, 0], x[:, :, 0], torch.zeros(1, 1), torch.zeros(1, 1),
                        torch.zeros(1, 1, 64, 64))


def test_chunked_grids_stay_within_one_launch(lib):
    """B*H*ceil(T/64) UT groups beyond one launch's grid limit return GDR_ERR_SHAPE (never a
    truncated grid), for every chunked entry point; the buffers sit 2^52 bytes apart so that no
    overlap check fires first."""
    P = [ctypes.c_void_p(i << 52) for i in range(1, 10)]
    B, T = 1 << 20, 1 << 22  # 2^21 state groups at d_v = 32, but 2^36 UT groups
    assert lib.gdr_chunk_fwd(B, 1, T, 128, 32, 0, 0, *P[:5], None, P[5], None, P[6], 1 << 20, None) == SHAPE
    assert lib.gdr_gdn2_chunk_fwd(B, 1, T, 128, 32, 0, *P[:6], None, P[6], None, P[7], 1 << 20, None) == SHAPE
    assert lib.gdr_chunk_fwd_fused_prep(B, 1, T, 128, 32, 0, *P[:7], None, P[7], None, P[8], 1 << 20, None) == SHAPE
    assert lib.gdr_gdp_chunk_fwd(B, 1, T // 2, 2, 128, 32, 0, *P[:5], None, P[5], None, P[6], 1 << 20, None) == SHAPE
