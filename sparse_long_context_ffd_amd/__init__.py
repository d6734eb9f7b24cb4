"""FFD sparse decode attention for MI355X (gfx950).

The hot path -- KV quantise/append, the fused scan -> Top-δ select -> attend
decode kernel, and the split combine -- is hand-written HIP behind the C ABI
in ``include/ffd.h`` (``libffd.so``, built in-tree). This package is its thin
Python binding; PyTorch provides device memory and streams.
"""

from .ffd import (  # noqa: F401
    EXPORTED_SYMBOLS,
    FFD_ERR_HIP,
    FFD_ERR_INVALID_ARG,
    FFD_ERR_UNSUPPORTED,
    FFD_ERR_WORKSPACE,
    FFD_OK,
    FFDError,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    alloc_workspace,
    decode,
    decode_multi,
    ffd_abi_version,
    ffd_combine,
    ffd_decode,
    ffd_decode_multi,
    ffd_decode_multi_workspace_bytes,
    ffd_decode_noalloc,
    ffd_decode_paged,
    ffd_decode_paged_multi,
    ffd_decode_partials,
    ffd_decode_thumb,
    ffd_decode_workspace_bytes,
    ffd_last_error,
    ffd_quantize_kv,
    ffd_quantize_kv_paged,
    ffd_quantize_kv_thumb,
    lib,
    quantize_kv,
    quantize_kv_thumb,
)
