"""MI355X (gfx950) fused multi-head attention: forward pass (dense and split-KV) and backward pass.

The computation lives in libfmha.so (hand-written HIP, C ABI in include/fmha.h); this
package only loads it and marshals arguments.
"""
from ._lib import (  # noqa: F401
    DTYPES,
    EXPORTS,
    LIB_PATH,
    MASKS,
    FmhaError,
    check,
    fmha_bwd,
    fmha_bwd_workspace_size,
    fmha_fwd,
    fmha_fwd_splitkv,
    fmha_fwd_splitkv_noalloc,
    fmha_fwd_splitkv_paged,
    fmha_paged_kv,
    fmha_paged_kv_append,
    fmha_fwd_splitkv_workspace_size,
    fmha_status_string,
    fmha_varlen,
    fmha_version,
    load,
    make_paged_kv,
    make_varlen,
)
