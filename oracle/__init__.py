"""fp64 CPU oracle for varlen, paged, GQA attention (TEST INFRASTRUCTURE ONLY).

This package is the parity authority for the HIP library in
``attention_cu_seqlens_amd``.  It is plain numpy in float64, slow and written to
be checked by eye against the pages it cites.  It shares no code, header, table
or helper with the HIP path, and it imports nothing from it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path never calls it.

Page key used in citations (the pages a reader has):
  [BLT]   facebookresearch/blt issue "Cross Attention does not work on CPU and
          older GPUs" -- the FlexAttention lowering arguments in its CPU traceback.
  [ORT]   onnxruntime PR "[CUDA] PagedAttention: add SM<80 fp16 fallback via
          memory-efficient attention" -- sections Implementation, Scratch
          allocation, Testing.
  [FLEX]  pytorch commit "[FlexAttention] Enforce Q,K,V memory layouts for fp8
          flex attention to avoid perf degradation" -- commit message (Context,
          Fix summary, Benchmarks), the test diff, ``_enforce_mem_layouts`` and
          the ``flex_attention`` docstring.
  [NANO]  nanochat issue "FA3 loader reports success on Blackwell (sm_120) then
          dies at first kernel launch" -- section "Note on impact".
  [VLLM]  vllm-project/flash-attention PR "Rope dim" -- review comments.

Parity status per function is listed in ``oracle.attention.PIN_STATUS``; every
function there is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_pins.py``
except where the entry says "parity unpinned".
"""

from .attention import (  # noqa: F401
    PIN_STATUS,
    MASK_CAUSAL,
    MASK_DOCUMENT,
    MASK_PATCH,
    cu_seqlens,
    reshape_and_cache,
    unpack_qkv,
    new_token_positions,
    rotary,
    rotary_reshape_and_cache,
    gather_paged,
    visibility,
    BlockMask,
    block_visibility,
    attention_varlen,
    attention_varlen_bwd,
    paged_attention,
    paged_decode,
    paged_decode_fp8kv,
    e4m3_decode,
    fp8_attention,
    default_scale,
)
