"""Exact fused attention for AMD MI355X (gfx950): Python binding of libattn.so.

The binding only marshals arguments: every step of attention runs in the HIP
kernels behind the C ABI declared in include/attn.h.  torch provides device
memory and the current stream.  There is no fallback: if the library is not
built, or no GPU is present, calls raise.
"""
from .binding import (  # noqa: F401
    AttnError,
    LIB_PATH,
    abi_version,
    attention,
    bwd,
    bwd_block_sparse,
    bwd_dkdv,
    bwd_dropout,
    bwd_dq,
    bwd_dq_fused,
    bwd_noalloc,
    bwd_noalloc_max_rows,
    bwd_preprocess,
    bwd_workspace_bytes,
    decode,
    decode_workspace_bytes,
    fwd,
    fwd_block_sparse,
    fwd_dropout,
    fwd_fp8,
    load_library,
    status_string,
)
