"""Python binding of libattn.so — fused softmax-attention forward for AMD MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/attn.h: every function here takes
torch tensors (device memory owned by the caller), checks dtype/rank/device, and passes data
pointers, element strides, sizes and the current HIP stream to the library entry point of the
same name. All arithmetic runs in the library's HIP kernels; there is no other code path.
If libattn.so has not been built, importing the bindings raises immediately.
"""

from __future__ import annotations

from ._lib import (  # noqa: F401
    AttnError,
    ATTN_OK,
    ATTN_ERR_INVALID_ARG,
    ATTN_ERR_UNSUPPORTED,
    ATTN_ERR_WORKSPACE,
    ATTN_ERR_LAUNCH,
    EXPORTED_SYMBOLS,
    lib_path,
    load_library,
    attn_fwd,
    attn_fwd_splitkv,
    attn_combine_lse,
    attn_fwd_decode,
    attn_decode_workspace_bytes,
    attn_fwd_decode_noalloc,
    ATTN_DECODE_SCRATCH_BYTES,
    attn_fwd_blocksparse,
    attn_splitkv_num_splits,
    attn_splitkv_workspace_bytes,
    attn_blocksparse_check,
    attn_fwd_vertical_slash,
    attn_vertical_slash_workspace_bytes,
    attn_vertical_slash_check,
    attn_build_sparse_index,
    attn_sparse_index_sizes,
    attn_sparse_index_workspace_bytes,
    attn_build_vslash_index,
    attn_status_string,
    attn_last_error,
    splitkv_decode,
)
