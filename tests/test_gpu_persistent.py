"""Equal-length batches at head size 64.  Under stored block lists such a
batch runs the persistent path (one workgroup per CU over a fixed snake of
tiles); without them it runs the four-wave workgroups like any other batch.

Each case is held to the oracle and, bit for bit, to the same call with one
more, empty, sequence appended (total_q then differs from batch *
max_seqlen_q, so the launcher takes its ragged-batch path: one workgroup per
tile).  A query row's arithmetic does not depend on which workgroup runs
it, so the two outputs must be identical.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (ATOL_16, DEV, REL_16, _i32, banner, compare, gpu_cache, lib_module,
                        oracle_prefill, requires_gpu, sample_rows)

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _run(A, w, cache, extra_empty, window=0, softcap=0.0, block_mask=None):
    """The prefill of w; with extra_empty, one empty sequence is appended
    (zero queries and keys, its block-table row a copy of the first)."""
    kc, vc, bt, _ = cache
    q_lens, kv_lens = list(w.q_lens), list(w.kv_lens)
    table = np.asarray(w.block_table)
    if extra_empty:
        q_lens.append(0)
        kv_lens.append(0)
        table = np.concatenate([table, table[:1]], axis=0)
    cu_q = A.attn_cu_seqlens(_i32(q_lens))
    cu_kv = A.attn_cu_seqlens(_i32(kv_lens))
    q_ids = None if w.q_ids is None else _i32(w.q_ids)
    kv_ids = None if w.kv_ids is None else _i32(w.kv_ids)
    args = (w.q.to(DEV).contiguous(), kc, vc, _i32(table), cu_q, cu_kv, int(max(q_lens)),
            int(max(kv_lens)))
    if block_mask is None:
        out, lse = A.attn_paged_prefill_fwd(*args, scale=w.scale, mask_flags=w.mask_flags,
                                            q_ids=q_ids, kv_ids=kv_ids, return_lse=True,
                                            window=window, softcap=softcap)
    else:
        qbs, kbs, kn, ki, fn, fi = block_mask
        if extra_empty:
            # one more sequence in the lists: no blocks listed
            kn = np.concatenate([kn, np.zeros_like(kn[:1])])
            ki = np.concatenate([ki, np.zeros_like(ki[:1])])
            fn = np.concatenate([fn, np.zeros_like(fn[:1])])
            fi = np.concatenate([fi, np.zeros_like(fi[:1])])
        out, lse = A.attn_paged_prefill_block_sparse_fwd(
            *args, qbs, kbs, _i32(kn), _i32(ki), _i32(fn), _i32(fi), scale=w.scale,
            mask_flags=w.mask_flags, q_ids=q_ids, kv_ids=kv_ids, return_lse=True, window=window,
            softcap=softcap)
    torch.cuda.synchronize()
    return out, lse


def _check(A, w, what, rows=None, window=0, softcap=0.0, block_mask=None):
    banner(f"persistent {what}: {len(w.q_lens)} x {int(w.q_lens[0])} tokens, "
           f"{w.num_heads}/{w.num_kv_heads} heads, flags {w.mask_flags}")
    cache = gpu_cache(w, A)
    out_p, lse_p = _run(A, w, cache, False, window, softcap, block_mask)
    out_d, lse_d = _run(A, w, cache, True, window, softcap, block_mask)
    assert torch.equal(out_p, out_d), f"{what}: persistent and dispatched outputs differ"
    assert torch.equal(lse_p, lse_d), f"{what}: persistent and dispatched LSE differ"
    bm = None if block_mask is None else block_mask
    ref_o, ref_l = oracle_prefill(w, rows, window=window, softcap=softcap, block_mask=bm)
    compare(out_p, lse_p, ref_o, ref_l, ATOL_16, REL_16, rows=rows, what=f"persistent_{what}")


def test_persistent_gqa_causal(A):
    lens = [777] * 6
    w = W.make_prefill("pc", 501, "bf16", lens, lens, 8, 2, 64, 16, W.MASK_CAUSAL)
    _check(A, w, "gqa_causal")


def test_persistent_patch_mask_f16(A):
    lens = [1500] * 4
    rng = np.random.default_rng(502)
    ids = []
    for n in lens:
        patch = np.repeat(np.arange(n), rng.integers(2, 15, n))[:n]
        ids.append(patch.astype(np.int32))
    ids = np.concatenate(ids)
    w = W.make_prefill("pp", 503, "f16", lens, [256] * 4, 4, 4, 64, 16, W.MASK_PATCH, q_ids=ids)
    _check(A, w, "patch")


def test_persistent_document_window_cap(A):
    lens = [900] * 5
    rng = np.random.default_rng(504)
    ids = np.concatenate([np.sort(rng.integers(0, 6, n)).astype(np.int32) for n in lens])
    w = W.make_prefill("pd", 505, "bf16", lens, lens, 8, 4, 64, 32,
                       W.MASK_DOCUMENT | W.MASK_CAUSAL, q_ids=ids, kv_ids=ids)
    _check(A, w, "document_window_cap", window=200, softcap=30.0)


def test_persistent_block_sparse(A):
    lens = [1024] * 3
    w = W.make_prefill("pb", 506, "bf16", lens, lens, 4, 2, 64, 16, W.MASK_CAUSAL)
    bm = (128, 128) + W.random_block_mask(np.random.default_rng(507), w.q_lens, w.kv_lens, 128,
                                           128, 1)
    _check(A, w, "block_sparse", block_mask=bm)


def test_persistent_many_tiles_per_workgroup(A):
    """24 x 2048 tokens, 16 heads without grouping: 3,072 query tiles, about 12
    per workgroup of each XCD's snake; sampled rows against the oracle."""
    lens = [2048] * 24
    w = W.make_prefill("pm", 508, "bf16", lens, lens, 16, 16, 64, 16, W.MASK_CAUSAL)
    rows = sample_rows(w.q_lens, 12, 509)
    _check(A, w, "many_tiles", rows=rows)


def test_persistent_fewer_tiles_than_workgroups(A):
    """Two 100-token sequences: fewer tiles than workgroups, most workgroups
    find no item."""
    lens = [100, 100]
    w = W.make_prefill("pf", 510, "bf16", lens, lens, 4, 1, 64, 16, W.MASK_CAUSAL)
    _check(A, w, "few_tiles")
