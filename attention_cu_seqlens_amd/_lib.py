"""ctypes view of libattn_cu_seqlens.so (the C ABI in include/attn_cu_seqlens.h).

Loading fails loudly if the library was not built: there is no fallback.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_cu_seqlens.so")

ATTN_OK = 0
STATUS_NAMES = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL_ARG",
    2: "ATTN_ERR_BAD_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_DEVICE",
    5: "ATTN_ERR_LAUNCH",
    6: "ATTN_ERR_WORKSPACE",
}
ATTN_F16, ATTN_BF16, ATTN_FP8_E4M3 = 0, 1, 2
ATTN_DECODE_SCRATCH_BYTES = 16 << 20   # attn_paged_decode_fwd_noalloc's scratch per GPU
MASK_NONE, MASK_CAUSAL, MASK_DOCUMENT, MASK_PATCH = 0, 1, 2, 4

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_size = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/attn_cu_seqlens.h
SIGNATURES = {
    "attn_abi_version": (ctypes.c_int, []),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_cu_seqlens": (ctypes.c_int, [_p, _p, _i32, _p]),
    "attn_reshape_and_cache": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32,
                                              _i32, _i32, _i32, ctypes.c_int, _p]),
    "attn_paged_prefill_fwd": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32,
                                              _i32, _i32, _i32, _i32, _i32, _i32, _f32, _u32,
                                              _p, _p, _i32, _f32, ctypes.c_int, _p, _p, _p]),
    "attn_varlen_bwd_workspace_bytes": (_size, [_i32, _i32]),
    "attn_varlen_bwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _f32, _u32, _p, _p, _i32, _f32,
                                       ctypes.c_int, _p, _p, _p, _p, _size, _p]),
    "attn_rotary_reshape_and_cache": (
        ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _p, _p, _p, _p, _i32, _p, _p,
                       _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p]),
    "attn_paged_prefill_block_sparse_fwd": (
        ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                       _i32, _i32, _f32, _u32, _p, _p, _i32, _f32, _i32, _i32, _i32, _i32, _i32,
                       _p, _p, _p, _p, ctypes.c_int, _p, _p, _p]),
    "attn_paged_decode_workspace_bytes": (_size, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "attn_paged_decode_fwd": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _f32, _i32, _f32, _i32, ctypes.c_int,
                                             _p, _p, _p, _size, _p]),
    "attn_paged_decode_fwd_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _i32, _i32, _i32,
                                                     _i32, _i32, _i32, _i32, _f32, _i32, _f32, _i32,
                                                     ctypes.c_int, _p, _p, _p]),
    "attn_paged_decode_fp8kv_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32,
                                                   _i32, _i32, _i32, _i32, _f32, _i32, _f32, _i32,
                                                   ctypes.c_int, _p, _p, _p, _size, _p]),
    "attn_fp8_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _f32, _u32, _p, _p, _i32, _f32, _p, _p, _p]),
}

_LIB = None


def load():
    """Load the library once and attach the C signatures."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m attention_cu_seqlens_amd.build_lib`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


class AttnError(RuntimeError):
    def __init__(self, func, status):
        self.status = status
        super().__init__(f"{func} returned {STATUS_NAMES.get(status, status)}")


def check(func, status):
    if status != ATTN_OK:
        raise AttnError(func, status)
