"""GPU parity of the paged prefill under a stored block-sparse mask against
the fp64 oracle.

The mask is the BlockMask of the blt issue's FlexAttention lowering arguments
(partial and full kv-block lists per query block) read per packed sequence;
the oracle's module docstring states the reading.  Bars as in
test_gpu_parity.py.  Cases: causal block lists (which must reproduce the
causal prefill), random lists with junk past each count for each mask-head
count (1, Hkv, Hq), the pages' single 2^30 block, element masks inside
partial blocks (document, window, q shorter than kv), fp16 with D = 64 and
the full-size varlen workload.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (ATOL_16, REL_16, banner, compare, gpu_cache, gpu_prefill,
                        gpu_prefill_sparse, lib_module, oracle_prefill, requires_gpu,
                        sample_rows, sub_workload)

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _case(A, w, bm, what, window=0, softcap=0.0, cache=None):
    banner(f"block-sparse {what}: q={w.q_lens.tolist()} kv={w.kv_lens.tolist()} "
           f"H={w.num_heads}/{w.num_kv_heads} D={w.head_size} blocks {bm[0]}x{bm[1]} "
           f"mask heads {bm[2].shape[1]} flags {w.mask_flags} {w.dtype}")
    out, lse = gpu_prefill_sparse(w, A, bm, cache=cache, window=window, softcap=softcap)
    ref_o, ref_l = oracle_prefill(w, window=window, softcap=softcap, block_mask=bm)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"sparse_{what}")
    return out, lse


def test_causal_block_lists_equal_causal_prefill(A):
    """Diagonal blocks partial, blocks below full, causal element mask: the
    result must be the causal prefill's, bit for bit."""
    w = W.make_prefill("bsc", 91, "bf16", [300, 200, 129], [300, 200, 129], 8, 2, 128, 16,
                       W.MASK_CAUSAL)
    cache = gpu_cache(w, A)
    kn, ki, fn, fi = W.causal_block_mask(w.q_lens, w.kv_lens, 128, 128)
    out, lse = _case(A, w, (128, 128, kn, ki, fn, fi), "causal_lists", cache=cache)
    out_c, lse_c = gpu_prefill(w, A, cache=cache)
    assert torch.equal(out, out_c)
    assert torch.equal(lse, lse_c)


@pytest.mark.parametrize("heads", ["one", "kv", "q"])
def test_random_lists_no_element_mask(A, heads):
    w = W.make_prefill("bsr", 92, "bf16", [333, 517, 64, 1], [333, 517, 64, 1], 8, 2, 128, 16,
                       0)
    hm = {"one": 1, "kv": 2, "q": 8}[heads]
    rng = np.random.default_rng(93)
    bm = (64, 64) + W.random_block_mask(rng, w.q_lens, w.kv_lens, 64, 64, hm)
    _case(A, w, bm, f"random_heads_{heads}")


def test_random_partial_only_causal_window(A):
    """Partial lists alone (no full pair), causal + window element mask,
    q shorter than kv, mask per query head with GQA 4."""
    w = W.make_prefill("bsw", 94, "bf16", [70, 260], [400, 520], 16, 4, 128, 32, W.MASK_CAUSAL)
    rng = np.random.default_rng(95)
    kn, ki, _, _ = W.random_block_mask(rng, w.q_lens, w.kv_lens, 32, 128, 16, p_partial=0.7,
                                       p_full=0.0)
    _case(A, w, (32, 128, kn, ki, None, None), "partial_causal_window", window=150)


def test_single_huge_block(A):
    """The pages' BlockMask: one block of 2^30 on each side.  Listed as
    partial it gives the element mask; listed as full it drops it."""
    w = W.make_prefill("bsh", 96, "bf16", [150, 77], [150, 77], 8, 8, 128, 16, W.MASK_CAUSAL)
    cache = gpu_cache(w, A)
    one = np.ones((2, 1, 1), np.int32)
    zero = np.zeros((2, 1, 1, 1), np.int32)
    out, _ = _case(A, w, (1 << 30, 1 << 30, one, zero, None, None), "huge_partial", cache=cache)
    assert torch.equal(out, gpu_prefill(w, A, cache=cache)[0])
    _case(A, w, (1 << 30, 1 << 30, 0 * one, zero, one, zero), "huge_full", cache=cache)


def test_document_mask_in_partial_blocks(A):
    rng = np.random.default_rng(97)
    lens = [420, 260]
    docs = []
    for n in lens:
        cuts = np.sort(rng.choice(np.arange(1, n), 3, replace=False))
        docs.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
    ids = np.concatenate(docs)
    w = W.make_prefill("bsd", 98, "bf16", lens, lens, 8, 4, 128, 16,
                       W.MASK_DOCUMENT | W.MASK_CAUSAL, q_ids=ids, kv_ids=ids)
    bm = (64, 128) + W.random_block_mask(rng, w.q_lens, w.kv_lens, 64, 128, 4, p_partial=0.6,
                                         p_full=0.2)
    _case(A, w, bm, "document_causal")


def test_d64_fp16_softcap(A):
    w = W.make_prefill("bs64", 99, "f16", [200, 95, 300], [200, 95, 300], 16, 2, 64, 32,
                       W.MASK_CAUSAL)
    rng = np.random.default_rng(100)
    bm = (128, 64) + W.random_block_mask(rng, w.q_lens, w.kv_lens, 128, 64, 2)
    _case(A, w, bm, "d64_fp16_softcap", softcap=3.0)


def test_full_varlen_causal_block_lists(A):
    """The varlen workload the benchmark times with FlexAttention-style causal
    block lists (128 x 128): sampled rows against the oracle, and the whole
    output against the causal prefill."""
    w = W.varlen_gqa_causal_bf16(device=DEV)
    banner(f"{w.name} block-sparse causal lists: total_q {w.total_q}")
    cache = gpu_cache(w, A)
    bm = (128, 128) + W.causal_block_mask(w.q_lens, w.kv_lens, 128, 128)
    out, lse = gpu_prefill_sparse(w, A, bm, cache=cache)
    out_c, lse_c = gpu_prefill(w, A, cache=cache)
    assert torch.equal(out, out_c)
    assert torch.equal(lse, lse_c)
    lens = np.asarray(w.q_lens)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 5})
    sub, q_idx = sub_workload(w, seqs)
    rows = sample_rows(sub.q_lens, 24, 101)
    sub_bm = (128, 128) + W.causal_block_mask(sub.q_lens, sub.kv_lens, 128, 128)
    ref_o, ref_l = oracle_prefill(sub, rows, block_mask=sub_bm)
    g = torch.as_tensor(q_idx[rows], device=out.device)
    compare(out[g], lse[g], ref_o[rows], ref_l[rows], ATOL_16, REL_16,
            what=f"{w.name} block-sparse seqs {seqs}")


@pytest.mark.parametrize("random_lists", [False, True])
def test_keys_beyond_one_page_window(A, random_lists):
    """kv_len 20000 at block size 16: the key range spans three chunks of
    512 pages, each compacted to its own listed tiles."""
    w = W.make_prefill("bslong", 136, "bf16", [200, 37], [20000, 9000], 8, 2, 128, 16,
                       W.MASK_CAUSAL)
    cache = gpu_cache(w, A)
    if random_lists:
        rng = np.random.default_rng(137)
        bm = (64, 64) + W.random_block_mask(rng, w.q_lens, w.kv_lens, 64, 64, 2, p_partial=0.2,
                                            p_full=0.2)
        _case(A, w, bm, "long_kv_random", cache=cache)
    else:
        bm = (128, 128) + W.causal_block_mask(w.q_lens, w.kv_lens, 128, 128)
        out, lse = _case(A, w, bm, "long_kv_causal_lists", cache=cache)
        out_c, lse_c = gpu_prefill(w, A, cache=cache)
        assert torch.equal(out, out_c) and torch.equal(lse, lse_c)


def test_every_block_hidden(A):
    """Empty lists everywhere: every row sees nothing (O = 0, LSE = -inf),
    whatever the element mask says."""
    w = W.make_prefill("bsnone", 142, "bf16", [130, 64], [130, 64], 8, 2, 128, 16, W.MASK_CAUSAL)
    kn, ki, fn, fi = W.causal_block_mask(w.q_lens, w.kv_lens, 64, 64)
    out, lse = _case(A, w, (64, 64, 0 * kn, ki, 0 * fn, fi), "every_block_hidden")
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_everything_at_once_d64_fp16(A):
    """Random partial / full lists per kv head, with a document mask, a
    window and a cap inside the partial blocks, fp16, D = 64."""
    rng = np.random.default_rng(149)
    lens = [333, 190]
    docs = []
    for n in lens:
        cuts = np.sort(rng.choice(np.arange(1, n), 2, replace=False))
        docs.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
    ids = np.concatenate(docs)
    w = W.make_prefill("bsall", 150, "f16", lens, lens, 8, 2, 64, 32,
                       W.MASK_DOCUMENT | W.MASK_CAUSAL, q_ids=ids, kv_ids=ids)
    bm = (64, 64) + W.random_block_mask(rng, w.q_lens, w.kv_lens, 64, 64, 2, p_partial=0.5,
                                        p_full=0.3)
    _case(A, w, bm, "everything_d64_fp16", window=90, softcap=4.0)
