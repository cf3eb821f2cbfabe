"""GPU parity of the local window and the score cap against the fp64 oracle.

The onnxruntime PR "[CUDA] PagedAttention: add SM<80 fp16 fallback via
memory-efficient attention" runs its parity matrix with "local window on/off"
and "softcap 0/50" (section Testing); the oracle's module docstring states how
both are read.  Bars as in test_gpu_parity.py.  The caps include the page's 50
(nearly linear for N(0,1) scores at scale 1/sqrt(D)) and small ones that bend
most scores, with a large scale so that many saturate.
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import (ATOL_16, ATOL_FP8, LSE_ATOL_FP8, REL_16, banner, compare, gpu_cache,
                        gpu_decode, gpu_fp8, gpu_prefill, lib_module, oracle_decode, oracle_fp8,
                        oracle_prefill, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _prefill_case(A, w, window, softcap, scale=None):
    banner(f"prefill window={window} softcap={softcap} q={w.q_lens.tolist()} "
           f"kv={w.kv_lens.tolist()} H={w.num_heads}/{w.num_kv_heads} D={w.head_size} "
           f"mask={w.mask_flags} {w.dtype}")
    if scale is not None:
        w.scale = scale
    out, lse = gpu_prefill(w, A, window=window, softcap=softcap)
    ref_o, ref_l = oracle_prefill(w, window=window, softcap=softcap)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16,
            what=f"prefill_w{window}_c{softcap}_{w.dtype}_d{w.head_size}")


@pytest.mark.parametrize("dtype,hq,hkv,d,window,softcap,scale", [
    ("bf16", 8, 2, 128, 100, 0.0, None),      # window alone, several key tiles
    ("bf16", 8, 2, 128, 0, 50.0, None),       # the page's cap
    ("bf16", 8, 2, 128, 0, 2.0, 0.5),         # a cap that bends and saturates
    ("f16", 4, 4, 64, 37, 3.0, 0.4),          # both, D = 64, fp16
    ("bf16", 16, 2, 64, 1, 0.0, None),        # window 1: each row sees its own key
])
def test_prefill_causal_window_softcap(A, dtype, hq, hkv, d, window, softcap, scale):
    w = W.make_prefill("wc", 61, dtype, [300, 200, 129], [300, 200, 129], hq, hkv, d, 16,
                       W.MASK_CAUSAL)
    _prefill_case(A, w, window, softcap, scale)


def test_prefill_window_without_causal_q_shorter(A):
    """Window alone (no causal flag) with q_len < kv_len: the lower bound
    follows the bottom-right position, keys to the right stay visible."""
    w = W.make_prefill("wq", 62, "bf16", [40, 130], [333, 400], 8, 2, 128, 16, W.MASK_NONE)
    _prefill_case(A, w, 90, 0.0)


def test_prefill_patch_mask_softcap(A):
    w = W.byte_patch_cross_bf16(batch=2, n_bytes=700, n_keys=96, seed=63)
    _prefill_case(A, w, 0, 1.5, 0.6)


def test_prefill_document_window(A):
    rng = np.random.default_rng(64)
    lens = [420, 260]
    docs = []
    for n in lens:
        cuts = np.sort(rng.choice(np.arange(1, n), 3, replace=False))
        docs.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
    ids = np.concatenate(docs)
    w = W.make_prefill("dw", 65, "bf16", lens, lens, 8, 4, 128, 16,
                       W.MASK_DOCUMENT | W.MASK_CAUSAL, q_ids=ids, kv_ids=ids)
    _prefill_case(A, w, 70, 0.0)


def test_decode_window_softcap(A):
    w = W.make_decode("dwc", 66, "bf16", [1, 17, 300, 1000, 2500, 0, 4096], 32, 8, 128, 16)
    cache = gpu_cache(w, A)
    for window, softcap in ((300, 0.0), (0, 4.0), (1000, 50.0), (1, 0.0)):
        banner(f"decode window={window} softcap={softcap}")
        ref_o, ref_l = oracle_decode(w, window=window, softcap=softcap)
        for st in (0, 256):
            out, lse = gpu_decode(w, A, split_tokens=st, cache=cache, window=window,
                                  softcap=softcap)
            compare(out, lse, ref_o, ref_l, ATOL_16, REL_16,
                    what=f"decode_w{window}_c{softcap}_split{st}")


def test_decode_d64_fp16_window_softcap(A):
    w = W.make_decode("dwc64", 67, "f16", [33, 700, 129], 16, 2, 64, 32)
    banner("decode d64 fp16 window 100 softcap 2")
    w.scale = 0.5
    out, lse = gpu_decode(w, A, window=100, softcap=2.0)
    ref_o, ref_l = oracle_decode(w, window=100, softcap=2.0)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="decode_d64_fp16_w100_c2")


@pytest.mark.parametrize("window,softcap", [(200, 0.0), (0, 3.0), (150, 50.0)])
def test_fp8_causal_window_softcap(A, window, softcap):
    w = W.make_fp8("fwc", 68, [1024, 640, 77], [1024, 640, 77], 8, 2, 128, W.MASK_CAUSAL)
    banner(f"fp8 window={window} softcap={softcap}")
    out, lse = gpu_fp8(w, A, window=window, softcap=softcap)
    ref_o, ref_l = oracle_fp8(w, window=window, softcap=softcap)
    compare(out, lse, ref_o, ref_l, ATOL_FP8, what=f"fp8_w{window}_c{softcap}",
            lse_atol=LSE_ATOL_FP8)
