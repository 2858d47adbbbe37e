"""MI355X (gfx950) fused exact attention: Python binding of libattn_mi355x.so.

The functions here only marshal arguments (tensor pointers, sizes, the current
HIP stream) into the C ABI of ``include/attn.h``; every step of the computation
runs in the library's HIP kernels.  Importing fails if the library has not been
built (``python exact_attention_108_amd/build.py``): there is no fallback path.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_F32,
    AttnError,
    LIB_PATH,
    attn_abi_version,
    attn_block_keep_from_bias,
    attn_bwd,
    attn_bwd_varlen,
    attn_bwd_workspace_bytes,
    attn_decode_paged,
    attn_decode_paged_fp8,
    attn_decode_paged_fp8_window,
    attn_decode_paged_alibi,
    attn_decode_paged_fp8_alibi,
    attn_decode_paged_noalloc,
    attn_decode_paged_window,
    DECODE_NOALLOC_MAX_BYTES,
    attn_decode_paged_workspace_bytes,
    attn_fwd,
    attn_fwd_fp8,
    attn_fwd_varlen,
    attn_prefill_paged,
    attn_prefill_paged_masked,
    attn_prefill_paged_fp8,
    attn_status_string,
    exported_symbols,
    pad_bias,
)
