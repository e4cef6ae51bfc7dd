"""FlashAttention forward for AMD MI355X (gfx950): HIP kernels behind a C ABI (include/fa.h).

`fa_fwd(q, k, v, mode=..., scale=..., mask=...)` runs the whole forward pass in libfa.so on
the GPU; `fa_fwd_lse` also returns each row's log-sum-exp; `pack_mask` turns a byte mask into
the bit layout of the bitmask mode and `mask_tiles` summarises a packed mask per 64 x 64 block.  The library is loaded on first
use, so `inputs` can be imported on machines without a GPU or a built library.
"""

from .fa import (FaError, fa_fwd, fa_fwd_ex_raw, fa_fwd_noalloc, fa_fwd_noalloc_raw, fa_fwd_lse, fa_fwd_lse_raw, fa_fwd_plan, fa_fwd_raw, fa_mask_tiles_raw,
                 fa_pack_mask_raw, fa_status_string, lib_path, load, mask_tiles, pack_mask,
                 set_kernel_events, workspace_bytes)

__all__ = ["fa_fwd", "fa_fwd_lse", "fa_fwd_plan", "fa_fwd_raw", "fa_fwd_lse_raw", "fa_fwd_ex_raw", "pack_mask", "mask_tiles",
           "fa_pack_mask_raw", "fa_mask_tiles_raw", "fa_status_string", "FaError", "lib_path",
           "load", "workspace_bytes", "fa_fwd_noalloc", "fa_fwd_noalloc_raw", "set_kernel_events"]
