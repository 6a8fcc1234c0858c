"""Split-KV decode attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libfd.so`` (HIP kernels behind the C ABI declared in
``include/fd.h``); ``binding`` marshals torch tensors into it. The library is
loaded on first use and its absence is an error, never a fallback.
"""
from .binding import (  # noqa: F401
    FdError,
    FdOptions,
    decode_plan,
    decode_workspace_size,
    device_num_cus,
    fd_decode,
    fd_decode_fp8kv,
    fd_paged_decode,
    fd_paged_decode_noalloc,
    fd_paged_decode_fp8kv,
    fd_prefill,
    lib,
    new_workspace,
    options,
    paged_plan,
    paged_workspace_size,
    prefill_flags,
    prefill_workspace_size,
    workspace_views,
)
