"""Exact attention forward (FlashAttention-2 order) for MI355X / gfx950.

The compute lives in libfa.so (HIP, built from csrc/ by ``build.build()``); this
package only marshals arguments to its C ABI (include/fa.h).
"""
from ._binding import (EXPORTED, FA_BF16, FA_F16, LIB_PATH, FaError, bwd, bwd_ex, fa_bwd, fa_bwd_ex,
                       fa_bwd_workspace_bytes,
                       fa_default_tile, fa_fwd, fa_fwd_ex, fa_fwd_split, fa_fwd_split_noalloc, fa_fwd_tiled, fa_split_default,
                       fa_split_workspace_bytes, fa_tile_supported, fwd, fwd_ex, fwd_split, fwd_split_noalloc, load_library,
                       status_str, SPLIT_SCRATCH_BYTES)

__all__ = ["fwd", "fwd_ex", "fwd_split", "fwd_split_noalloc", "fa_fwd_split_noalloc", "SPLIT_SCRATCH_BYTES", "bwd", "bwd_ex", "fa_bwd", "fa_bwd_ex", "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_tiled", "fa_fwd_ex", "fa_fwd_split",
           "fa_split_workspace_bytes", "fa_split_default", "fa_tile_supported", "fa_default_tile", "status_str",
           "load_library", "FaError", "FA_F16", "FA_BF16", "LIB_PATH", "EXPORTED"]
