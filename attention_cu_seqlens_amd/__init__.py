"""attention_cu_seqlens_amd: varlen, paged, GQA attention forward for MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C ABI
(include/attn_cu_seqlens.h, built into libattn_cu_seqlens.so).  This package
is the thin Python binding: the functions below only check and marshal torch
tensors (device memory and the current stream) into that ABI.
"""

from ._lib import (  # noqa: F401
    AttnError,
    ATTN_F16,
    ATTN_BF16,
    ATTN_FP8_E4M3,
    ATTN_DECODE_SCRATCH_BYTES,
    MASK_NONE,
    MASK_CAUSAL,
    MASK_DOCUMENT,
    MASK_PATCH,
)
from .api import (  # noqa: F401
    attn_cu_seqlens,
    attn_reshape_and_cache,
    attn_rotary_reshape_and_cache,
    attn_paged_prefill_fwd,
    attn_paged_prefill_block_sparse_fwd,
    attn_paged_decode_workspace_bytes,
    attn_paged_decode_fwd,
    attn_paged_decode_fwd_noalloc,
    attn_paged_decode_fp8kv_fwd,
    attn_fp8_fwd,
    attn_varlen_bwd,
    attn_varlen_bwd_workspace_bytes,
    library_path,
)
