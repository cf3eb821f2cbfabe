"""The allocation-free decode entry point against the workspace one.

attn_paged_decode_fwd_noalloc runs the decode kernels with their split
partials in the library's per-GPU scratch array instead of a caller
workspace.  Through the C ABI it must give the same bits as
attn_paged_decode_fwd on the same inputs and split size, on two calls in a
row where the second is smaller (the scratch keeps the first call's
partials, which the second must not read), and both stay within the parity
bars of the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (ATOL_16, REL_16, banner, compare, gpu_cache, lib_module, oracle_decode,
                        requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _both(A, w, split, window=0):
    kc, vc, bt, cu_kv = gpu_cache(w, A)
    q = w.q.to(DEV).contiguous()
    mskv = int(w.kv_lens.max(initial=0))
    out_n = torch.empty_like(q)
    lse_n = torch.empty((w.batch, w.num_heads), dtype=torch.float32, device=DEV)
    A.attn_paged_decode_fwd_noalloc(q, kc, vc, bt, cu_kv, mskv, scale=w.scale,
                                    split_tokens=split, window=window, out=out_n, lse=lse_n)
    torch.cuda.synchronize()
    out_w, lse_w = A.attn_paged_decode_fwd(q, kc, vc, bt, cu_kv, mskv, scale=w.scale,
                                           split_tokens=split, return_lse=True, window=window)
    torch.cuda.synchronize()
    return out_n, lse_n, out_w, lse_w


def test_noalloc_decode_two_calls_second_smaller(A):
    big = W.make_decode("na1", 501, "bf16", np.random.default_rng(502).integers(1, 20000, 48),
                        32, 8, 128, 16)
    small = W.make_decode("na2", 503, "bf16", [1, 0, 700, 3000, 257], 16, 2, 64, 16)
    for w, split, window in ((big, 1024, 0), (small, 256, 500)):
        banner(f"noalloc decode {w.name}: batch {w.batch}, H {w.num_heads}/{w.num_kv_heads}, "
               f"D {w.head_size}, split {split}, window {window}")
        out_n, lse_n, out_w, lse_w = _both(A, w, split, window)
        assert torch.equal(out_n, out_w), "noalloc output differs from the workspace call"
        assert torch.equal(lse_n, lse_w), "noalloc LSE differs from the workspace call"
        if w is small:
            ref_o, ref_l = oracle_decode(w, window=window)
            compare(out_n, lse_n, ref_o, ref_l, ATOL_16, REL_16, what="noalloc small")


def test_noalloc_decode_automatic_split_full_workload(A):
    """The paged GQA decode workload (64 sequences up to 32K keys) fits the
    scratch with the automatic split."""
    w = W.paged_gqa_decode_bf16(device=DEV)
    banner(f"noalloc decode {w.name}")
    out_n, lse_n, out_w, lse_w = _both(A, w, 0)
    assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)
