"""Bit-exact visibility probes for every mask kind, through the C ABI.

With scale = 0 every visible key of a row weighs exactly 1 (every score is
0), and with V_j = onehot(j mod D) the output row is the histogram of the
row's visible keys by residue divided by their number n:
O_i[d] = #{visible j : j mod D = d} / n_i and LSE_i = ln n_i.  Rounding
O_i[d] * n_i to the nearest integer recovers every residue count exactly
while each count stays below 256 (the 16-bit output carries 8 or more
significant bits), so the visible set that the kernels used is compared
count for count with the oracle's (oracle.visibility /
oracle.block_visibility); rows with no visible key must give zeros and
-inf.  This is the mask pin of the survey's oracle section: a single key
too many or too few on a row of a thousand keys changes a count, while it
moves the ordinary outputs by far less than their float bars.

Masks probed: causal with GQA row packing and q shorter than kv; document
(alone and with causal, ids absent on the key side); the byte->patch mask
of the blt issue "Cross Attention does not work on CPU and older GPUs"
(issue body: flex_attention under a block_mask); the local window with and
without causal, q shorter than kv ("local window on/off" of the
onnxruntime PR "[CUDA] PagedAttention: add SM<80 fp16 fallback via
memory-efficient attention", Testing); stored block lists (partial and
full, junk ids) for mask heads 1, Hkv and Hq (the FlexAttention lowering
arguments kv_num_blocks / kv_indices / full_kv_*); decode with a window
across split boundaries; and the fp8 kernel (one-hot V code 0x38 = 1.0).
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as ORC
import workloads as W
from gpu_common import (banner, gpu_decode, gpu_fp8, gpu_prefill, gpu_prefill_sparse,
                        lib_module, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _positions(lens):
    """Each token's index within its sequence, for the concatenated tokens."""
    return np.concatenate([np.arange(int(n)) for n in lens]) if np.sum(lens) else \
        np.zeros(0, dtype=np.int64)


def _onehot_tokens(kv_lens, hkv, d, dtype):
    """[total_kv, Hkv, D]: token j of its sequence is onehot(j mod D) in every head."""
    pos = _positions(kv_lens)
    v = torch.zeros((len(pos), hkv, d), dtype=torch.float32)
    if len(pos):
        v[torch.arange(len(pos)), :, torch.as_tensor(pos % d)] = 1.0
    return v.to(dtype)


def _check_rows(got, lse, vis, d, what):
    """got [q_len, D] float64, lse [q_len]; vis [q_len, kv_len] the oracle's
    visible set for these rows."""
    n = vis.sum(axis=1)
    onehot = np.zeros((vis.shape[1], d), dtype=np.int64)
    onehot[np.arange(vis.shape[1]), np.arange(vis.shape[1]) % d] = 1
    counts = vis.astype(np.int64) @ onehot
    assert counts.max(initial=0) < 256, "probe too large to be exact"
    rec = np.rint(got * n[:, None])
    bad = np.nonzero(~np.all(rec == counts, axis=1))[0]
    assert bad.size == 0, (f"{what}: visible set differs on rows {bad[:8].tolist()}: "
                           f"n={n[bad[:3]].tolist()}")
    empty = n == 0
    assert np.all(got[empty] == 0.0), f"{what}: a row without keys is not zero"
    assert np.all(np.isneginf(lse[empty])), f"{what}: a row without keys has a finite LSE"
    if (~empty).any():
        err = np.abs(lse[~empty] - np.log(n[~empty]))
        assert err.max() < 1e-5 * max(1.0, math.log(n.max())), f"{what}: LSE != ln n"
        # each output within one unit in the last place of its 16-bit value
        ref = counts[~empty] / n[~empty, None]
        ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
        assert np.all(np.abs(got[~empty] - ref) <= ulp), f"{what}: output beyond 1 ulp"
    return int(n.sum())


def _probe_prefill(A, w, what, window=0, block_mask=None):
    """Run the paged prefill on one-hot V at scale 0 and compare each
    (sequence, head)'s visible sets with the oracle's."""
    w = dataclasses.replace(w, v_new=_onehot_tokens(w.kv_lens, w.num_kv_heads, w.head_size,
                                                     w.v_new.dtype))
    banner(f"probe {what}: q={w.q_lens.tolist()[:6]} kv={w.kv_lens.tolist()[:6]} "
           f"H={w.num_heads}/{w.num_kv_heads} D={w.head_size} flags={w.mask_flags} W={window}")
    if block_mask is None:
        out, lse = gpu_prefill(w, A, scale=0.0, window=window)
    else:
        w0 = dataclasses.replace(w, scale=0.0)
        out, lse = gpu_prefill_sparse(w0, A, block_mask, window=window)
    o = out.float().cpu().double().numpy()
    ls = lse.cpu().double().numpy()
    cu_q = ORC.cu_seqlens(w.q_lens)
    cu_kv = ORC.cu_seqlens(w.kv_lens)
    total = 0
    for b in range(w.batch):
        ql, kl = int(w.q_lens[b]), int(w.kv_lens[b])
        if ql == 0:
            continue
        qi = None if w.q_ids is None else np.asarray(w.q_ids)[cu_q[b]:cu_q[b + 1]]
        ki = None if w.kv_ids is None else np.asarray(w.kv_ids)[cu_kv[b]:cu_kv[b + 1]]
        elem = ORC.visibility(ql, kl, w.mask_flags, qi, ki, window)
        for h in range(w.num_heads):
            vis = elem
            if block_mask is not None:
                qbs, kbs, kn, kidx, fn, fidx = block_mask
                hm = kn.shape[1]
                mh = 0 if hm == 1 else (h if hm == w.num_heads else
                                        h // (w.num_heads // w.num_kv_heads))
                vis = ORC.block_visibility(elem, qbs, kbs, kn[b, mh], kidx[b, mh],
                                           None if fn is None else fn[b, mh],
                                           None if fidx is None else fidx[b, mh])
            rows = slice(cu_q[b], cu_q[b + 1])
            total += _check_rows(o[rows, h], ls[rows, h], vis, w.head_size,
                                 f"{what} seq {b} head {h}")
    print(f"[probe] {what}: {total} visible (query, key) pairs match", flush=True)


# ---------------------------------------------------------------- prefill

@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 4)])
def test_probe_causal_gqa_q_shorter(A, hq, hkv):
    w = W.make_prefill("pc", 201, "bf16", [70, 300, 1, 129], [90, 300, 200, 1000], hq, hkv, 64,
                       16, W.MASK_CAUSAL)
    _probe_prefill(A, w, f"causal_gqa{hq // hkv}")


def _docs(rng, lens, n_cuts):
    out = []
    for n in lens:
        cuts = np.sort(rng.choice(np.arange(1, n), min(n_cuts, n - 1), replace=False))
        out.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
    return np.concatenate(out)


@pytest.mark.parametrize("flags", [W.MASK_DOCUMENT, W.MASK_DOCUMENT | W.MASK_CAUSAL])
def test_probe_document(A, flags):
    rng = np.random.default_rng(202)
    lens = [260, 190, 33]
    ids = _docs(rng, lens, 6)
    w = W.make_prefill("pd", 203, "bf16", lens, lens, 8, 2, 64, 16, flags, q_ids=ids, kv_ids=ids)
    _probe_prefill(A, w, f"document_{flags}")


def test_probe_document_q_shorter_unmatched_ids(A):
    """Queries are the last tokens of each sequence; the key-side documents
    carry even ids, and one run of query rows an odd id that no key has
    (those rows see nothing).  Ids stay non-decreasing within a sequence."""
    rng = np.random.default_rng(204)
    kv_lens, q_lens = [300, 220], [90, 220]
    kv_ids = 2 * _docs(rng, kv_lens, 5)
    cu = np.concatenate([[0], np.cumsum(kv_lens)])
    q_ids = np.concatenate([kv_ids[cu[b + 1] - q_lens[b]:cu[b + 1]] for b in range(2)])
    q_ids = np.where(q_ids == 4, 5, q_ids).astype(np.int32)
    assert (q_ids == 5).any()
    for flags in (W.MASK_DOCUMENT, W.MASK_DOCUMENT | W.MASK_CAUSAL):
        w = W.make_prefill("pdu", 205, "bf16", q_lens, kv_lens, 8, 4, 64, 16, flags,
                           q_ids=q_ids, kv_ids=kv_ids.astype(np.int32))
        _probe_prefill(A, w, f"document_unmatched_{flags}")


def test_probe_patch(A):
    """The byte->patch cross mask with the config-4 id recipe (patch lengths
    2..14); 96 patch keys, so late bytes see every key and short sequences
    leave keys unreachable."""
    w = W.byte_patch_cross_bf16(batch=3, n_bytes=700, n_keys=96, seed=206)
    _probe_prefill(A, w, "patch")


def test_probe_patch_more_keys_than_patches(A):
    w = W.byte_patch_cross_bf16(batch=2, n_bytes=300, n_keys=200, seed=207)
    _probe_prefill(A, w, "patch_unreachable_keys")


@pytest.mark.parametrize("flags,window", [(W.MASK_NONE, 37), (W.MASK_NONE, 1),
                                          (W.MASK_CAUSAL, 37), (W.MASK_CAUSAL, 300),
                                          (W.MASK_CAUSAL | W.MASK_DOCUMENT, 50)])
def test_probe_window(A, flags, window):
    q_lens, kv_lens = [50, 130, 7, 200], [400, 131, 300, 200]
    ids = None
    if flags & W.MASK_DOCUMENT:
        q_lens = kv_lens
        ids = _docs(np.random.default_rng(208), kv_lens, 4)
    w = W.make_prefill("pw", 209, "bf16", q_lens, kv_lens, 8, 2, 64, 16, flags, q_ids=ids,
                       kv_ids=ids)
    _probe_prefill(A, w, f"window{window}_flags{flags}", window=window)


@pytest.mark.parametrize("hm", [1, 2, 8])
def test_probe_block_lists(A, hm):
    """Random partial / full block lists with junk ids past each count; the
    element mask inside partial blocks is causal (document + causal for one
    head count)."""
    lens = [333, 517, 64, 1]
    flags, ids = W.MASK_CAUSAL, None
    if hm == 2:
        flags |= W.MASK_DOCUMENT
        ids = _docs(np.random.default_rng(210), lens[:3], 4)
        ids = np.concatenate([ids, np.zeros(1, np.int32)])
    w = W.make_prefill("pb", 211, "bf16", lens, lens, 8, 2, 64, 16, flags, q_ids=ids, kv_ids=ids)
    rng = np.random.default_rng(212 + hm)
    bm = (64, 128) + W.random_block_mask(rng, w.q_lens, w.kv_lens, 64, 128, hm)
    _probe_prefill(A, w, f"block_lists_hm{hm}", block_mask=bm)


def test_probe_block_lists_partial_only_window(A):
    w = W.make_prefill("pbw", 213, "bf16", [70, 260], [400, 520], 16, 4, 64, 32, W.MASK_CAUSAL)
    rng = np.random.default_rng(214)
    kn, ki, _, _ = W.random_block_mask(rng, w.q_lens, w.kv_lens, 32, 64, 16, p_partial=0.7,
                                       p_full=0.0)
    _probe_prefill(A, w, "block_lists_partial_window", window=150,
                   block_mask=(32, 64, kn, ki, None, None))


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("window,split", [(0, 256), (700, 256), (300, 512), (5000, 1024)])
def test_probe_decode_window_splits(A, window, split):
    lens = [1, 17, 300, 1000, 2500, 0, 4096, 700]
    w = W.make_decode("pdec", 215, "bf16", lens, 16, 2, 64, 16)
    w = dataclasses.replace(w, scale=0.0,
                            v_new=_onehot_tokens(w.kv_lens, w.num_kv_heads, 64, w.v_new.dtype))
    banner(f"probe decode window {window} split {split}")
    out, lse = gpu_decode(w, A, split_tokens=split, window=window)
    o = out.float().cpu().double().numpy()
    ls = lse.cpu().double().numpy()
    for b, kl in enumerate(lens):
        vis = ORC.visibility(1, kl, 0, window=window)
        for h in range(w.num_heads):
            _check_rows(o[b:b + 1, h], ls[b:b + 1, h], vis, 64, f"decode seq {b} head {h}")


# ---------------------------------------------------------------- fp8

@pytest.mark.parametrize("flags,window", [(W.MASK_CAUSAL, 0), (W.MASK_DOCUMENT | W.MASK_CAUSAL, 0),
                                          (W.MASK_NONE, 45), (W.MASK_CAUSAL, 130)])
def test_probe_fp8(A, flags, window):
    q_lens, kv_lens = [300, 77, 513], [300, 77, 513]
    ids = None
    if flags & W.MASK_DOCUMENT:
        ids = _docs(np.random.default_rng(216), kv_lens, 6)
    if window and not flags & W.MASK_CAUSAL:
        q_lens = [100, 77, 13]
    w = W.make_fp8("p8", 217, q_lens, kv_lens, 8, 2, 128, flags, q_ids=ids, kv_ids=ids)
    pos = _positions(w.kv_lens)
    v8 = torch.zeros((w.num_kv_heads, 128, len(pos)), dtype=torch.uint8)
    v8[:, torch.as_tensor(pos % 128), torch.arange(len(pos))] = 0x38   # e4m3 1.0
    w = dataclasses.replace(w, scale=0.0, v8_colmajor=v8,
                            descale=np.asarray([w.descale[0], w.descale[1], 1.0], np.float32))
    banner(f"probe fp8 flags {flags} window {window}")
    out, lse = gpu_fp8(w, A, window=window)
    o = out.float().cpu().double().numpy()
    ls = lse.cpu().double().numpy()
    cu_q, cu_kv = ORC.cu_seqlens(w.q_lens), ORC.cu_seqlens(w.kv_lens)
    for b in range(w.batch):
        ql, kl = int(w.q_lens[b]), int(w.kv_lens[b])
        qi = None if ids is None else ids[cu_q[b]:cu_q[b + 1]]
        ki = None if ids is None else ids[cu_kv[b]:cu_kv[b + 1]]
        vis = ORC.visibility(ql, kl, flags, qi, ki, window)
        for h in range(w.num_heads):
            _check_rows(o[cu_q[b]:cu_q[b + 1], h], ls[cu_q[b]:cu_q[b + 1], h], vis, 128,
                        f"fp8 seq {b} head {h}")
