"""libgdr: the gated delta rule on AMD Instinct MI355X (gfx950).

Python face of the C ABI in include/gdr.h.  ``chunk_fwd`` runs the chunkwise
forward pass and returns (o, final_state) (the UT kernel over all chunks, then the
chunk-serial state kernel; the workspace is the caller's tensor or one allocated with
torch); ``chunk_fwd_fused_prep`` runs it from raw
projections (normalisation and gates fused in); ``gdp_chunk_fwd`` is the same pass
for the Gated Delta Product (n_h key/value/beta substeps per token) and
``gdn2_chunk_fwd`` for Gated DeltaNet-2 (separate erase and write gates);
``frame_fwd`` runs the frame-level implicit update (tokens in unordered frames);
``decode_step`` advances resident states by one token in place.  The HIP
library is loaded on first use and its absence is an error: there is no CPU
fallback.
"""
from ._binding import (EXPORTED_SYMBOLS, LIBRARY_PATH, NOALLOC_WORKSPACE_BYTES, GdrError, chunk_fwd,
                       chunk_fwd_fused_prep, chunk_fwd_noalloc,
                       chunk_fwd_fused_prep_workspace_size,
                       chunk_fwd_workspace_size, decode_step, frame_fwd, frame_fwd_workspace_size, gdn2_chunk_fwd,
                       gdn2_chunk_fwd_workspace_size, gdp_chunk_fwd, gdp_chunk_fwd_workspace_size, load_library, status_string, version)

__all__ = ["chunk_fwd", "chunk_fwd_workspace_size", "chunk_fwd_noalloc", "NOALLOC_WORKSPACE_BYTES", "chunk_fwd_fused_prep", "chunk_fwd_fused_prep_workspace_size", "frame_fwd", "frame_fwd_workspace_size", "gdp_chunk_fwd", "gdp_chunk_fwd_workspace_size", "gdn2_chunk_fwd", "gdn2_chunk_fwd_workspace_size", "decode_step", "GdrError", "load_library", "version", "status_string",
           "LIBRARY_PATH", "EXPORTED_SYMBOLS"]
