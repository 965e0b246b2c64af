"""libgdr: the gated delta rule on AMD Instinct MI355X (gfx950).

Python face of the C ABI in include/gdr.h.  ``chunk_fwd`` runs the chunkwise
forward pass and returns (o, final_state); ``decode_step`` advances resident
states by one token in place.  The HIP library is loaded on first use and its
absence is an error: there is no CPU fallback.
"""
from ._binding import (EXPORTED_SYMBOLS, LIBRARY_PATH, GdrError, chunk_fwd, decode_step, load_library,
                       status_string, version)

__all__ = ["chunk_fwd", "decode_step", "GdrError", "load_library", "version", "status_string",
           "LIBRARY_PATH", "EXPORTED_SYMBOLS"]
