"""Exact tiled attention (prefill and KV-cache decode) for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI (include/fa.h,
built as exact_tiled_attention_prefill_amd/libfa.so).  This package is the thin
Python layer over that ABI: it marshals torch device tensors into pointers and
the current HIP stream.  Importing it does not load the library; the first call
does, and fails loudly if the library has not been built.
"""

from .binding import (  # noqa: F401
    FaError,
    decode,
    decode_noalloc,
    decode_paged,
    decode_paged_workspace_bytes,
    decode_workspace_bytes,
    library_path,
    load_library,
    prefill,
    prefill_backward,
    prefill_backward_workspace_bytes,
    prefill_varlen,
)
