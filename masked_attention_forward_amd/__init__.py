"""Masked scaled-dot-product attention forward for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libfa.so`` (hand-written HIP kernels); this package
only marshals arguments to it. Loading is lazy: importing the package does not need a GPU,
and every entry point raises if the library is missing.
"""

from .binding import (  # noqa: F401
    FA_LAYOUTS,
    FaError,
    fa_fwd,
    fa_fwd_workspace_size,
    fa_mask_probe,
    fa_plan_stats,
    fa_status_str,
    fa_tile_shape,
    flash_attention,
    library_path,
    load_library,
)
