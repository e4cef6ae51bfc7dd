"""FlashAttention forward for AMD MI355X (gfx950): HIP kernels behind a C ABI (include/fa.h).

`fa_fwd(q, k, v, mode=..., scale=..., mask=...)` runs the whole forward pass in libfa.so on
the GPU; `fa_fwd_lse` also returns each row's log-sum-exp.  The library is loaded on first
use, so `inputs` can be imported on machines without a GPU or a built library.
"""

from .fa import (FaError, fa_fwd, fa_fwd_lse, fa_fwd_lse_raw, fa_fwd_raw, fa_status_string,
                 lib_path, load)

__all__ = ["fa_fwd", "fa_fwd_lse", "fa_fwd_raw", "fa_fwd_lse_raw", "fa_status_string", "FaError",
           "lib_path", "load"]
