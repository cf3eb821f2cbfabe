"""Helpers for the GPU parity tests: run a workload through the C ABI (via the
binding) and through the oracle, and compare.

The oracle side and the HIP side each compute their own cu_seqlens and fill
their own paged cache from the same generated tokens.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as ORC

ATOL_16 = 2e-2     # max-abs bound for fp16 / bf16 outputs against the fp64 oracle
REL_16 = 1e-2      # relative L2 bound
ATOL_FP8 = 6e-2    # max-abs bound for fp8 outputs
LSE_ATOL = 2e-3    # fp32 logsumexp of exactly the same inputs
# fp8: the row normaliser is summed from probabilities rounded to e4m3, whose
# round-to-nearest-even relative error is at most 2^-4 (3 mantissa bits), so
# ln(l) -- and the LSE -- may move by up to ln(1 + 2^-4) < 2^-4.
LSE_ATOL_FP8 = 2.0 ** -4

DEV = "cuda"


def gpu_available():
    try:
        return torch.cuda.is_available()
    except Exception:
        return False


def lib_module():
    import attention_cu_seqlens_amd as A
    A._lib.load()
    return A


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------- oracle side

def oracle_prefill(w, rows=None, window=0, softcap=0.0, block_mask=None):
    cu_q = ORC.cu_seqlens(w.q_lens)
    cu_kv = ORC.cu_seqlens(w.kv_lens)
    cu_new = ORC.cu_seqlens(w.new_lens)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    kc = np.full(shape, np.nan)
    vc = np.full(shape, np.nan)
    k = w.k_new.double().cpu().numpy()
    v = w.v_new.double().cpu().numpy()
    kc, vc = ORC.reshape_and_cache(k, v, kc, vc, w.block_table, cu_new, cu_kv, w.block_size)
    q = w.q.double().cpu().numpy()
    return ORC.paged_attention(q, kc, vc, w.block_table, cu_q, cu_kv, w.block_size, w.scale,
                               w.mask_flags, w.q_ids, w.kv_ids, rows, window, softcap,
                               None if block_mask is None else ORC.BlockMask(*block_mask))


def oracle_decode(w, batches=None, window=0, softcap=0.0):
    cu_kv = ORC.cu_seqlens(w.kv_lens)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    kc = np.full(shape, np.nan)
    vc = np.full(shape, np.nan)
    k = w.k_new.double().cpu().numpy()
    v = w.v_new.double().cpu().numpy()
    kc, vc = ORC.reshape_and_cache(k, v, kc, vc, w.block_table, cu_kv, cu_kv, w.block_size)
    q = w.q.double().cpu().numpy()
    return ORC.paged_decode(q, kc, vc, w.block_table, cu_kv, w.block_size, w.scale, batches,
                            window, softcap)


def oracle_decode_fp8kv(w, batches=None, window=0, softcap=0.0):
    """Decode over the workload's fp8 cache: codes placed by the oracle's
    reshape_and_cache into a cache of NaN codes (0x7F)."""
    cu_kv = ORC.cu_seqlens(w.kv_lens)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    kc = np.full(shape, 0x7F, dtype=np.uint8)
    vc = np.full(shape, 0x7F, dtype=np.uint8)
    kc, vc = ORC.reshape_and_cache(w.k_new.cpu().numpy(), w.v_new.cpu().numpy(), kc, vc,
                                   w.block_table, cu_kv, cu_kv, w.block_size)
    q = w.q.double().cpu().numpy()
    return ORC.paged_decode_fp8kv(q, kc, vc, w.kv_descale, w.block_table, cu_kv, w.block_size,
                                  w.scale, batches, window, softcap)


def oracle_fp8(w, rows=None, window=0, softcap=0.0):
    cu_q = ORC.cu_seqlens(w.q_lens)
    cu_kv = ORC.cu_seqlens(w.kv_lens)
    return ORC.fp8_attention(w.q.cpu().numpy(), w.k_new.cpu().numpy(),
                             w.v8_colmajor.cpu().numpy(), w.descale, cu_q, cu_kv, w.scale,
                             w.mask_flags, w.q_ids, w.kv_ids, rows, window, softcap)


# ------------------------------------------------------------------- GPU side

def _i32(a):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32).to(DEV)


def gpu_cache(w, A, poison=float("nan")):
    """Cu-seqlens and a NaN-poisoned paged cache filled through the library."""
    cu_kv = A.attn_cu_seqlens(_i32(w.kv_lens))
    cu_new = A.attn_cu_seqlens(_i32(w.new_lens))
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    dt = w.k_new.dtype
    kc = torch.full(shape, poison, dtype=dt, device=DEV)
    vc = torch.full(shape, poison, dtype=dt, device=DEV)
    bt = _i32(w.block_table)
    A.attn_reshape_and_cache(w.k_new.to(DEV).contiguous(), w.v_new.to(DEV).contiguous(), kc, vc,
                             bt, cu_new, cu_kv)
    return kc, vc, bt, cu_kv


def gpu_prefill(w, A, cache=None, scale=None, block_table=None, window=0, softcap=0.0):
    kc, vc, bt, cu_kv = cache if cache is not None else gpu_cache(w, A)
    if block_table is not None:
        bt = _i32(block_table)
    cu_q = A.attn_cu_seqlens(_i32(w.q_lens))
    q_ids = None if w.q_ids is None else _i32(w.q_ids)
    kv_ids = None if w.kv_ids is None else _i32(w.kv_ids)
    out, lse = A.attn_paged_prefill_fwd(
        w.q.to(DEV).contiguous(), kc, vc, bt, cu_q, cu_kv, int(w.q_lens.max(initial=0)),
        int(w.kv_lens.max(initial=0)), scale=w.scale if scale is None else scale,
        mask_flags=w.mask_flags, q_ids=q_ids, kv_ids=kv_ids, return_lse=True, window=window,
        softcap=softcap)
    torch.cuda.synchronize()
    return out, lse


def gpu_prefill_sparse(w, A, block_mask, cache=None, window=0, softcap=0.0):
    """block_mask: (q_block, kv_block, kv_num, kv_idx, full_num, full_idx),
    numpy arrays (the full pair may be None)."""
    kc, vc, bt, cu_kv = cache if cache is not None else gpu_cache(w, A)
    qbs, kbs, kn, ki, fn, fi = block_mask
    cu_q = A.attn_cu_seqlens(_i32(w.q_lens))
    q_ids = None if w.q_ids is None else _i32(w.q_ids)
    kv_ids = None if w.kv_ids is None else _i32(w.kv_ids)
    out, lse = A.attn_paged_prefill_block_sparse_fwd(
        w.q.to(DEV).contiguous(), kc, vc, bt, cu_q, cu_kv, int(w.q_lens.max(initial=0)),
        int(w.kv_lens.max(initial=0)), qbs, kbs, _i32(kn), _i32(ki),
        None if fn is None else _i32(fn), None if fi is None else _i32(fi), scale=w.scale,
        mask_flags=w.mask_flags, q_ids=q_ids, kv_ids=kv_ids, return_lse=True, window=window,
        softcap=softcap)
    torch.cuda.synchronize()
    return out, lse


def gpu_decode(w, A, split_tokens=0, cache=None, window=0, softcap=0.0):
    kc, vc, bt, cu_kv = cache if cache is not None else gpu_cache(w, A)
    out, lse = A.attn_paged_decode_fwd(w.q.to(DEV).contiguous(), kc, vc, bt, cu_kv,
                                       int(w.kv_lens.max(initial=0)), scale=w.scale,
                                       split_tokens=split_tokens, return_lse=True, window=window,
                                       softcap=softcap)
    torch.cuda.synchronize()
    return out, lse


def gpu_decode_fp8kv(w, A, split_tokens=0, cache=None, window=0, softcap=0.0):
    """Decode over the workload's fp8 cache, written by the library into a
    cache poisoned with NaN codes."""
    kc, vc, bt, cu_kv = cache if cache is not None else gpu_cache(w, A, poison=0x7F)
    ds = torch.as_tensor(w.kv_descale, dtype=torch.float32).to(DEV)
    out, lse = A.attn_paged_decode_fp8kv_fwd(w.q.to(DEV).contiguous(), kc, vc, ds, bt, cu_kv,
                                             int(w.kv_lens.max(initial=0)), scale=w.scale,
                                             split_tokens=split_tokens, return_lse=True,
                                             window=window, softcap=softcap)
    torch.cuda.synchronize()
    return out, lse


def gpu_fp8(w, A, window=0, softcap=0.0):
    cu_q = A.attn_cu_seqlens(_i32(w.q_lens))
    cu_kv = A.attn_cu_seqlens(_i32(w.kv_lens))
    q_ids = None if w.q_ids is None else _i32(w.q_ids)
    kv_ids = None if w.kv_ids is None else _i32(w.kv_ids)
    out, lse = A.attn_fp8_fwd(w.q.to(DEV), w.k_new.to(DEV), w.v8_colmajor.to(DEV),
                              torch.as_tensor(w.descale, dtype=torch.float32).to(DEV), cu_q,
                              cu_kv, int(w.q_lens.max()), int(w.kv_lens.max()), scale=w.scale,
                              mask_flags=w.mask_flags, q_ids=q_ids, kv_ids=kv_ids,
                              return_lse=True, window=window, softcap=softcap)
    torch.cuda.synchronize()
    return out, lse


# ------------------------------------------------------------ random draws

def draw_masked_lengths(rng, batch, max_kv, max_q, masks):
    """One random varlen layout: kv lengths in [1, max_kv) with some empty
    sequences, a mask from `masks` and query lengths and ids that fit it --
    document ids cut each sequence at a few points (queries = keys), patch ids
    are non-decreasing indices below the key count, causal query blocks end at
    each key range's end (bottom-right), no mask takes any query lengths.
    A draw with no query token or no key at all is drawn again from the same
    generator (whole-batch empty inputs have tests of their own), so every
    random case runs.  Returns (mask, q_lens, kv_lens, q_ids, kv_ids)."""
    import workloads as W
    mask = int(rng.choice(masks))
    kv_lens = rng.integers(1, max_kv, batch)
    kv_lens[rng.random(batch) < 0.15] = 0
    q_ids = kv_ids = None
    if mask & W.MASK_DOCUMENT:
        q_lens = kv_lens.copy()
        docs = []
        for n in kv_lens:
            cuts = np.sort(rng.integers(1, max(2, int(n)), int(rng.integers(0, 4))))
            docs.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
        q_ids = kv_ids = np.concatenate(docs).astype(np.int32)
    elif mask & W.MASK_PATCH:
        q_lens = rng.integers(0, max_q, batch)
        q_ids = np.concatenate([np.sort(rng.integers(0, max(1, int(k)), int(n)))
                                for n, k in zip(q_lens, kv_lens)]).astype(np.int32)
    elif mask & W.MASK_CAUSAL:
        q_lens = np.array([int(rng.integers(0, int(k) + 1)) for k in kv_lens])
    else:
        q_lens = rng.integers(0, max_q, batch)
    if int(np.sum(q_lens)) == 0 or int(np.sum(kv_lens)) == 0:
        return draw_masked_lengths(rng, batch, max_kv, max_q, masks)
    return mask, np.asarray(q_lens), kv_lens, q_ids, kv_ids


# ----------------------------------------------------------------- comparison

def compare(out_gpu, lse_gpu, out_ref, lse_ref, atol, rel=None, rows=None, what="",
            lse_atol=LSE_ATOL):
    """Element-wise comparison on (optionally) sampled rows; returns error stats."""
    o = out_gpu.float().cpu().double().numpy()
    l = lse_gpu.cpu().double().numpy()
    if rows is not None:
        o, l, out_ref, lse_ref = o[rows], l[rows], out_ref[rows], lse_ref[rows]
    assert not np.any(np.isnan(o)), f"{what}: NaN in GPU output"
    diff = np.abs(o - out_ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    denom = float(np.linalg.norm(out_ref))
    rel_l2 = float(np.linalg.norm(o - out_ref) / denom) if denom > 0 else 0.0
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), inf_ref), f"{what}: fully-masked rows differ"
    lse_err = float(np.max(np.abs(l[~inf_ref] - lse_ref[~inf_ref]))) if (~inf_ref).any() else 0.0
    stats = dict(max_abs=max_abs, rel_l2=rel_l2, lse_err=lse_err)
    print(f"[parity] {what}: {stats}", flush=True)
    assert max_abs <= atol, f"{what}: max-abs {max_abs} > {atol}"
    if rel is not None:
        assert rel_l2 <= rel, f"{what}: rel-L2 {rel_l2} > {rel}"
    assert lse_err <= lse_atol, f"{what}: LSE error {lse_err}"
    return stats


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs a GPU")


# ------------------------------------------------------- sampled full-size runs

def sub_workload(w, seqs, decode=False):
    """The sequences `seqs` of a paged workload, alone: the same tokens and
    ids, their pages renumbered 0..n-1 in order.  Lets the oracle check
    sampled outputs of a full-size GPU run without building the whole cache
    in fp64 (placement does not change the result: the oracle's permutation
    pin).  Returns (sub, q_index) where q_index[i] is the row of w holding
    row i of sub."""
    assert np.array_equal(w.new_lens, w.kv_lens)
    seqs = [int(b) for b in seqs]
    cq = np.concatenate([[0], np.cumsum(w.q_lens, dtype=np.int64)])
    ck = np.concatenate([[0], np.cumsum(w.kv_lens, dtype=np.int64)])
    bs = w.block_size
    nblk = [(int(w.kv_lens[b]) + bs - 1) // bs for b in seqs]
    table = np.zeros((len(seqs), max(1, max(nblk))), dtype=np.int32)
    nxt = 0
    for i, n in enumerate(nblk):
        table[i, :n] = np.arange(nxt, nxt + n)
        nxt += n
    kv_idx = np.concatenate([np.arange(ck[b], ck[b + 1]) for b in seqs])
    if decode:
        q_idx = np.asarray(seqs, dtype=np.int64)
    else:
        q_idx = np.concatenate([np.arange(cq[b], cq[b + 1]) for b in seqs])
    tq = torch.as_tensor(q_idx, device=w.q.device)
    tk = torch.as_tensor(kv_idx, device=w.k_new.device)
    import dataclasses
    sub = dataclasses.replace(
        w, q_lens=w.q_lens[seqs].copy(), kv_lens=w.kv_lens[seqs].copy(),
        new_lens=w.new_lens[seqs].copy(), num_blocks=max(1, nxt), block_table=table,
        q_ids=None if w.q_ids is None else np.asarray(w.q_ids)[q_idx],
        kv_ids=None if w.kv_ids is None else np.asarray(w.kv_ids)[kv_idx],
        q=w.q[tq].cpu(), k_new=w.k_new[tk].cpu(), v_new=w.v_new[tk].cpu(), extra={})
    return sub, q_idx


def sub_fp8(w, seqs):
    """fp8 counterpart of sub_workload (dense, V column-major)."""
    seqs = [int(b) for b in seqs]
    cq = np.concatenate([[0], np.cumsum(w.q_lens, dtype=np.int64)])
    ck = np.concatenate([[0], np.cumsum(w.kv_lens, dtype=np.int64)])
    q_idx = np.concatenate([np.arange(cq[b], cq[b + 1]) for b in seqs])
    kv_idx = np.concatenate([np.arange(ck[b], ck[b + 1]) for b in seqs])
    tq = torch.as_tensor(q_idx, device=w.q.device)
    tk = torch.as_tensor(kv_idx, device=w.k_new.device)
    import dataclasses
    sub = dataclasses.replace(
        w, q_lens=w.q_lens[seqs].copy(), kv_lens=w.kv_lens[seqs].copy(),
        new_lens=w.new_lens[seqs].copy(), block_table=w.block_table[seqs].copy(),
        q_ids=None if w.q_ids is None else np.asarray(w.q_ids)[q_idx],
        kv_ids=None if w.kv_ids is None else np.asarray(w.kv_ids)[kv_idx],
        q=w.q[tq].cpu(), k_new=w.k_new[tk].cpu(),
        v8_colmajor=w.v8_colmajor[:, :, tk].cpu(), extra={})
    return sub, q_idx


def sample_rows(q_lens, per_seq, seed):
    """Row indices (within the concatenated sequences) to check: each
    sequence's first two rows, its middle and last row, and `per_seq` more
    drawn at random."""
    rng = np.random.default_rng(seed)
    rows, base = [], 0
    for n in (int(x) for x in q_lens):
        if n:
            pick = {0, min(1, n - 1), n // 2, n - 1}
            pick |= set(rng.choice(n, size=min(per_seq, n), replace=False).tolist())
            rows += [base + i for i in sorted(pick)]
        base += n
    return np.asarray(rows, dtype=np.int64)
