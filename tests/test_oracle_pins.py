"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``check_*`` function takes the oracle module and raises AssertionError on
a mismatch.  The tests run them on the real oracle; ``test_planted_mistakes``
plants plausible mistakes into the oracle (on the CPU) and requires that at
least one check catches each of them.

Sources of truth used here (none of them is the oracle's own formula):
  * values the pages print (tests/golden/*.json, each with its citation);
  * hand-derived closed forms (tests/golden/two_key_example.json, uniform
    scores give the mean of the visible V rows, LSE = ln(count));
  * library routines for special cases: numpy.cumsum, numpy.tril, torch CPU
    float64 scaled_dot_product_attention (dense, GQA, explicit masks),
    torch.logsumexp, torch.float8_e4m3fn decoding;
  * invariants: block-table permutation, score shifts, GQA head expansion,
    varlen packing, decode = last causal row.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as ORC

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa(q, k, v, scale, is_causal=False, attn_mask=None, enable_gqa=False):
    """torch CPU float64 SDPA on one sequence; q [L, Hq, D], k/v [S, Hkv, D]."""
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    K = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    V = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if attn_mask is None else torch.from_numpy(attn_mask)
    o = F.scaled_dot_product_attention(Q, K, V, attn_mask=m, is_causal=is_causal, scale=scale,
                                       enable_gqa=enable_gqa)
    return o[0].permute(1, 0, 2).numpy()


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# check functions (each raises AssertionError on mismatch)
# ----------------------------------------------------------------------------

def check_default_scale(A):
    g = _golden("flex_lowering_args.json")
    E = g["query_shape_BHLE"][-1]
    assert A.default_scale(E) == g["scale"]


def check_cu_seqlens_golden(A):
    for case in _golden("cu_seqlens_examples.json")["cases"]:
        got = A.cu_seqlens(case["lens"])
        assert got.dtype == np.int32
        assert got.tolist() == case["cu"], (case, got)


def check_cu_seqlens_cumsum(A):
    rng = np.random.default_rng(7)
    for n in (1, 2, 17, 300):
        lens = rng.integers(0, 5000, n)
        ref = np.concatenate([[0], np.cumsum(lens)])
        assert np.array_equal(A.cu_seqlens(lens), ref)


def check_reshape_and_cache_golden(A):
    g = _golden("reshape_and_cache_example.json")
    bs, nb = g["block_size"], g["num_blocks"]
    table = np.asarray(g["block_table"], dtype=np.int32)
    kv_lens, new_lens = g["kv_lens"], g["new_lens"]
    vals = np.asarray(g["new_token_values"], dtype=np.int64)
    k_new = vals.reshape(-1, 1, 1)
    cache = np.full((nb, bs, 1, 1), g["untouched_value"], dtype=np.int64)
    cu_new = np.concatenate([[0], np.cumsum(new_lens)])
    cu_kv = np.concatenate([[0], np.cumsum(kv_lens)])
    kc, vc = A.reshape_and_cache(k_new, -k_new, cache, cache, table, cu_new, cu_kv, bs)
    exp = np.asarray(g["expected_cache"], dtype=np.int64)
    assert np.array_equal(kc[:, :, 0, 0], exp), kc[:, :, 0, 0]
    expv = np.where(exp == g["untouched_value"], exp, -exp)
    assert np.array_equal(vc[:, :, 0, 0], expv)


def check_reshape_gather_roundtrip(A):
    """Scatter then gather returns the new tokens bit for bit; other slots keep their poison."""
    rng = np.random.default_rng(11)
    bs, hkv, d = 4, 2, 3
    kv_lens = np.array([5, 0, 9, 4])
    new_lens = np.array([2, 0, 9, 1])
    need = [(n + bs - 1) // bs for n in kv_lens]
    nb = sum(need) + 2
    perm = rng.permutation(nb)
    table = np.full((4, max(need)), nb - 1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    poison = np.int64(-(2**40))
    cache = np.full((nb, bs, hkv, d), poison, dtype=np.int64)
    total_new = int(new_lens.sum())
    k_new = rng.integers(0, 2**30, (total_new, hkv, d))
    v_new = rng.integers(0, 2**30, (total_new, hkv, d))
    cu_new = np.concatenate([[0], np.cumsum(new_lens)])
    cu_kv = np.concatenate([[0], np.cumsum(kv_lens)])
    kc, vc = A.reshape_and_cache(k_new, v_new, cache, cache, table, cu_new, cu_kv, bs)
    written = 0
    for b in range(4):
        gk = A.gather_paged(kc, table[b], int(kv_lens[b]), bs)
        gv = A.gather_paged(vc, table[b], int(kv_lens[b]), bs)
        n, L = int(new_lens[b]), int(kv_lens[b])
        assert np.array_equal(gk[L - n:], k_new[cu_new[b]:cu_new[b + 1]])
        assert np.array_equal(gv[L - n:], v_new[cu_new[b]:cu_new[b + 1]])
        assert np.all(gk[:L - n] == poison)
        written += n
    assert int(np.sum(kc != poison)) == written * hkv * d


def check_gather_identity_and_permutation(A):
    """Identity placement equals the packed layout; any placement gathers the same tokens."""
    rng = np.random.default_rng(3)
    bs, hkv, d, L = 4, 2, 3, 13
    packed = _rand(rng, L, hkv, d)
    nb = (L + bs - 1) // bs
    cache = np.full((nb, bs, hkv, d), np.nan)
    for j in range(L):
        cache[j // bs, j % bs] = packed[j]
    ident = np.arange(nb)
    assert np.array_equal(A.gather_paged(cache, ident, L, bs), packed)
    perm = rng.permutation(nb)
    cache2 = np.full_like(cache, np.nan)
    cache2[perm] = cache
    assert np.array_equal(A.gather_paged(cache2, perm, L, bs), packed)


def check_visibility_page_predicate(A):
    g = _golden("causal_mask_predicate.json")
    L = g["shape_BHLE"][2]
    vis = A.visibility(L, L, ORC.MASK_CAUSAL)
    brute = np.array([[q_idx >= kv_idx for kv_idx in range(L)] for q_idx in range(L)])
    assert np.array_equal(vis, brute)
    assert int(vis.sum()) == g["visible_pairs_per_head"]


def check_visibility_closed_forms(A):
    # bottom-right causal with q_len != kv_len is a shifted lower triangle
    for q_len, kv_len in ((5, 9), (9, 5), (1, 7), (7, 7), (3, 0)):
        vis = A.visibility(q_len, kv_len, ORC.MASK_CAUSAL)
        assert np.array_equal(vis, np.tril(np.ones((q_len, kv_len), bool), k=kv_len - q_len))
    # PATCH with patch index = byte index and equal lengths is causal
    n = 11
    assert np.array_equal(A.visibility(n, n, ORC.MASK_PATCH, np.arange(n)),
                          np.tril(np.ones((n, n), bool)))
    # PATCH: each byte sees keys 0..patch(byte)
    pid = np.array([0, 0, 1, 1, 1, 2, 4, 4])
    vis = A.visibility(len(pid), 6, ORC.MASK_PATCH, pid)
    assert vis.sum(axis=1).tolist() == [1, 1, 2, 2, 2, 3, 5, 5]
    # DOCUMENT is block diagonal over runs of equal ids
    docs = np.array([0, 0, 0, 1, 1, 2, 2, 2, 2])
    blocks = [np.ones((3, 3)), np.ones((2, 2)), np.ones((4, 4))]
    bd = np.zeros((9, 9), bool)
    o = 0
    for blk in blocks:
        n_ = blk.shape[0]
        bd[o:o + n_, o:o + n_] = True
        o += n_
    assert np.array_equal(A.visibility(9, 9, ORC.MASK_DOCUMENT, docs, docs), bd)
    assert np.array_equal(A.visibility(9, 9, ORC.MASK_DOCUMENT | ORC.MASK_CAUSAL, docs, docs),
                          bd & np.tril(np.ones((9, 9), bool)))


def check_two_key_golden(A):
    g = _golden("two_key_example.json")
    q = np.asarray(g["q"])[:, None, :]
    k = np.asarray(g["k"])[:, None, :]
    v = np.asarray(g["v"])[:, None, :]
    out, lse = A.attention_varlen(q, k, v, [0, 1], [0, 2], g["scale"])
    assert np.allclose(out[0, 0], g["out"], rtol=0, atol=1e-15), out
    assert abs(lse[0, 0] - g["lse"]) < 1e-15


def check_dense_vs_sdpa(A):
    """Dense single sequence, no GQA: causal and full, against torch SDPA fp64."""
    rng = np.random.default_rng(5)
    L, H, D = 23, 3, 8
    q, k, v = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    for flags, causal in ((0, False), (ORC.MASK_CAUSAL, True)):
        out, _ = A.attention_varlen(q, k, v, [0, L], [0, L], 0.37, flags)
        ref = _sdpa(q, k, v, 0.37, is_causal=causal)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def check_gqa_vs_sdpa(A):
    rng = np.random.default_rng(6)
    L, HQ, HKV, D = 17, 8, 2, 4
    q, k, v = _rand(rng, L, HQ, D), _rand(rng, L, HKV, D), _rand(rng, L, HKV, D)
    out, _ = A.attention_varlen(q, k, v, [0, L], [0, L], 0.5, ORC.MASK_CAUSAL)
    ref = _sdpa(q, k, v, 0.5, is_causal=True, enable_gqa=True)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    # explicit expansion gives the same answer through the oracle itself
    kx = np.repeat(k, HQ // HKV, axis=1)
    vx = np.repeat(v, HQ // HKV, axis=1)
    out2, _ = A.attention_varlen(q, kx, vx, [0, L], [0, L], 0.5, ORC.MASK_CAUSAL)
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-13)


def check_varlen_bottom_right_vs_sdpa(A):
    """Packed varlen with q_len != kv_len: each sequence equals SDPA with the shifted-tril mask."""
    rng = np.random.default_rng(8)
    q_lens, kv_lens = [3, 7, 1, 6], [8, 7, 5, 6]
    HQ, HKV, D = 4, 2, 5
    cu_q = np.concatenate([[0], np.cumsum(q_lens)])
    cu_k = np.concatenate([[0], np.cumsum(kv_lens)])
    q = _rand(rng, cu_q[-1], HQ, D)
    k = _rand(rng, cu_k[-1], HKV, D)
    v = _rand(rng, cu_k[-1], HKV, D)
    out, lse = A.attention_varlen(q, k, v, cu_q, cu_k, 0.3, ORC.MASK_CAUSAL)
    for b in range(4):
        ql, kl = q_lens[b], kv_lens[b]
        mask = np.tril(np.ones((ql, kl), bool), k=kl - ql)
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        ref = _sdpa(q[qs], k[ks], v[ks], 0.3, attn_mask=mask, enable_gqa=True)
        assert np.allclose(out[qs], ref, rtol=1e-12, atol=1e-12), b
        # LSE against torch.logsumexp of the masked, scaled scores
        kx = np.repeat(k[ks], HQ // HKV, axis=1)
        s = 0.3 * np.einsum("ihd,jhd->hij", q[qs], kx)
        s = np.where(mask[None], s, -np.inf)
        ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy().T
        assert np.allclose(lse[qs], ref_lse, rtol=1e-12, atol=1e-12), b


def check_uniform_scores_mean(A):
    """scale = 0: every visible key gets the same weight, O = mean of visible V, LSE = ln(count)."""
    rng = np.random.default_rng(9)
    L, H, D = 12, 2, 6
    q, k, v = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    out, lse = A.attention_varlen(q, k, v, [0, L], [0, L], 0.0, ORC.MASK_CAUSAL)
    for i in range(L):
        assert np.allclose(out[i], v[:i + 1].mean(axis=0), rtol=1e-13, atol=1e-13)
        assert abs(lse[i, 0] - math.log(i + 1)) < 1e-13


def check_single_key_rows(A):
    """Causal row 0 sees only key 0: its output is V[0] exactly."""
    rng = np.random.default_rng(10)
    q_lens = [4, 9]
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    q, k, v = _rand(rng, 13, 2, 4), _rand(rng, 13, 1, 4), _rand(rng, 13, 1, 4)
    out, lse = A.attention_varlen(q, k, v, cu, cu, 0.8, ORC.MASK_CAUSAL)
    for b in range(2):
        r = cu[b]
        for h in range(2):
            assert np.array_equal(out[r, h], v[r, 0])
            assert math.isclose(lse[r, h], 0.8 * float(q[r, h] @ k[r, 0]), rel_tol=1e-14,
                                abs_tol=1e-15)


def check_shift_invariance(A):
    """Adding a per-row constant to every score leaves O unchanged and shifts LSE by it."""
    rng = np.random.default_rng(12)
    L, H, D = 10, 2, 4
    q, k, v = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    c = rng.standard_normal((L, H, 1))
    q2 = np.concatenate([q, c], axis=2)
    k2 = np.concatenate([k, np.ones((L, H, 1))], axis=2)
    out1, lse1 = A.attention_varlen(q, k, v, [0, L], [0, L], 0.6, ORC.MASK_CAUSAL)
    out2, lse2 = A.attention_varlen(q2, k2, v, [0, L], [0, L], 0.6, ORC.MASK_CAUSAL)
    assert np.allclose(out1, out2, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse2 - lse1, 0.6 * c[:, :, 0], rtol=1e-12, atol=1e-12)


def check_fully_masked_rows(A):
    """No visible key: O = 0 and LSE = -inf, never NaN (empty sequence and unmatched document)."""
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 5, 1, 3), _rand(rng, 4, 1, 3), _rand(rng, 4, 1, 3)
    out, lse = A.attention_varlen(q, k, v, [0, 2, 5], [0, 0, 4], 1.0, ORC.MASK_DOCUMENT,
                                  q_ids=np.array([0, 0, 1, 9, 2]), kv_ids=np.array([1, 1, 2, 2]))
    assert np.all(out[0:2] == 0) and np.all(np.isneginf(lse[0:2]))   # kv_len = 0
    assert np.all(out[3] == 0) and np.isneginf(lse[3, 0])              # doc 9 has no key
    assert np.allclose(out[2], _sdpa(q[2:3], k[0:2], v[0:2], 1.0)[0], rtol=1e-12, atol=1e-12)
    assert np.allclose(out[4], _sdpa(q[4:5], k[2:4], v[2:4], 1.0)[0], rtol=1e-12, atol=1e-12)
    assert not np.any(np.isnan(out))


def check_paged_equals_packed(A):
    """Paged attention over a permuted pool equals packed attention on the same tokens."""
    rng = np.random.default_rng(14)
    bs, HQ, HKV, D = 4, 4, 2, 3
    lens = np.array([6, 1, 11])
    cu = np.concatenate([[0], np.cumsum(lens)])
    k = _rand(rng, cu[-1], HKV, D)
    v = _rand(rng, cu[-1], HKV, D)
    q = _rand(rng, cu[-1], HQ, D)
    need = [(n + bs - 1) // bs for n in lens]
    nb = sum(need) + 1
    perm = rng.permutation(nb - 1)
    table = np.full((3, max(need)), nb - 1, dtype=np.int32)
    kc = np.full((nb, bs, HKV, D), np.nan)
    vc = np.full((nb, bs, HKV, D), np.nan)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
        for j in range(lens[b]):
            kc[table[b, j // bs], j % bs] = k[cu[b] + j]
            vc[table[b, j // bs], j % bs] = v[cu[b] + j]
    out_p, lse_p = A.paged_attention(q, kc, vc, table, cu, cu, bs, 0.4, ORC.MASK_CAUSAL)
    out_r, lse_r = A.attention_varlen(q, k, v, cu, cu, 0.4, ORC.MASK_CAUSAL)
    assert np.array_equal(out_p, out_r) and np.array_equal(lse_p, lse_r)
    assert not np.any(np.isnan(out_p))
    for b in range(3):
        L = lens[b]
        ref = _sdpa(q[cu[b]:cu[b + 1]], k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]], 0.4,
                    is_causal=True, enable_gqa=True)
        assert np.allclose(out_p[cu[b]:cu[b + 1]], ref, rtol=1e-12, atol=1e-12), L


def check_decode_is_last_causal_row(A):
    rng = np.random.default_rng(15)
    bs, HQ, HKV, D = 8, 4, 1, 5
    lens = np.array([9, 17, 1])
    cu = np.concatenate([[0], np.cumsum(lens)])
    need = [(n + bs - 1) // bs for n in lens]
    nb = sum(need)
    table = np.zeros((3, max(need)), dtype=np.int32)
    kc = np.zeros((nb, bs, HKV, D))
    vc = np.zeros((nb, bs, HKV, D))
    perm = rng.permutation(nb)
    off = 0
    k = _rand(rng, cu[-1], HKV, D)
    v = _rand(rng, cu[-1], HKV, D)
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
        for j in range(lens[b]):
            kc[table[b, j // bs], j % bs] = k[cu[b] + j]
            vc[table[b, j // bs], j % bs] = v[cu[b] + j]
    q_full = _rand(rng, cu[-1], HQ, D)
    last = cu[1:] - 1
    out_d, lse_d = A.paged_decode(q_full[last], kc, vc, table, cu, bs, 0.45)
    for b in range(3):
        ref = _sdpa(q_full[cu[b]:cu[b + 1]], k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]], 0.45,
                    is_causal=True, enable_gqa=True)
        assert np.allclose(out_d[b], ref[-1], rtol=1e-12, atol=1e-12)


def check_e4m3_table(A):
    codes = np.arange(256, dtype=np.uint8)
    got = A.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    g = _golden("e4m3_values.json")
    for code, val in g["values"].items():
        x = A.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert x == val and np.signbit(x) == np.signbit(val), (code, x, val)
    for code in g["nan_codes"]:
        assert np.isnan(A.e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0])


def check_fp8_attention(A):
    """fp8: the two-key example through e4m3 codes and descales, and a random case
    against SDPA on the values torch decodes from the same codes."""
    # two keys: k0 = 0, k1 = (1,0,...) with descale 1; q = (ln2-ish): use scale = ln 2
    one, zero = 0x38, 0x00
    q8 = np.array([[[one, zero, zero, zero]]], dtype=np.uint8)             # q = (1,0,0,0)
    k8 = np.array([[[zero] * 4], [[one, zero, zero, zero]]], dtype=np.uint8)
    three = 0x44  # 1.5 * 2^1 = 3
    v_rows = np.array([[three, zero, zero, zero], [zero, three, zero, zero]], dtype=np.uint8)
    v8 = v_rows.T[None]                                                      # [1, 4, 2]
    out, lse = A.fp8_attention(q8, k8, v8, (1.0, 1.0, 1.0), [0, 1], [0, 2], math.log(2.0))
    assert np.allclose(out[0, 0], [1.0, 2.0, 0.0, 0.0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0] - math.log(3.0)) < 1e-15
    # random, descaled, GQA, causal
    rng = np.random.default_rng(16)
    L, HQ, HKV, D = 9, 4, 2, 8
    codes = lambda *s: rng.integers(0, 256, s, dtype=np.uint8) & np.uint8(0xF7)  # no NaN codes
    q8, k8, vr = codes(L, HQ, D), codes(L, HKV, D), codes(L, HKV, D)
    ds = (0.5, 0.25, 2.0)
    v8 = np.ascontiguousarray(vr.transpose(1, 2, 0))
    out, _ = A.fp8_attention(q8, k8, v8, ds, [0, L], [0, L], 0.1, ORC.MASK_CAUSAL)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = _sdpa(ds[0] * dec(q8), ds[1] * dec(k8), ds[2] * dec(vr), 0.1, is_causal=True,
                enable_gqa=True)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def check_decode_fp8kv(A):
    """fp8 paged cache: a hand-derived two-key example whose dk and dv differ
    (so a swap shows), a constant-V closed form, and a random paged case
    against decode over caches that torch decodes from the same codes."""
    one, two, nan_code = 0x38, 0x40, 0x7F
    # page 1 holds the sequence, page 0 is NaN codes that must never be read
    kc = np.full((2, 2, 1, 4), nan_code, dtype=np.uint8)
    vc = np.full((2, 2, 1, 4), nan_code, dtype=np.uint8)
    kc[1, 0, 0] = [one, 0, 0, 0]       # k0 = dk * (1, 0, 0, 0)
    kc[1, 1, 0] = 0                    # k1 = 0
    vc[1, 0, 0] = one                  # v0 = dv * 1
    vc[1, 1, 0] = two                  # v1 = dv * 2
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    dk, dv, scale = 2.0 * math.log(3.0), 0.5, 0.5
    # scores: scale * dk = ln 3 and 0, weights 3/4 and 1/4
    out, lse = A.paged_decode_fp8kv(q, kc, vc, (dk, dv), np.array([[1]]), [0, 2], 2, scale)
    assert np.allclose(out[0, 0], 0.75 * 0.5 + 0.25 * 1.0, rtol=0, atol=1e-14), out
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14
    # any keys, every V code 2.0: each output is exactly 2 dv
    rng = np.random.default_rng(17)
    bs, HQ, HKV, D = 4, 4, 2, 8
    lens = np.array([7, 1, 10])
    cu = np.concatenate([[0], np.cumsum(lens)])
    nb = 8
    table = np.array([[5, 2, 0], [7, 0, 0], [1, 6, 3]], dtype=np.int32)
    kc = rng.integers(0, 256, (nb, bs, HKV, D), dtype=np.uint8) & np.uint8(0xF7)
    vc = np.full((nb, bs, HKV, D), two, dtype=np.uint8)
    q = _rand(rng, 3, HQ, D)
    out, _ = A.paged_decode_fp8kv(q, kc, vc, (0.3, 0.25), table, cu, bs, 0.2)
    assert np.allclose(out, 0.5, rtol=0, atol=1e-14)
    # random V, window and cap: decode over the torch-decoded, descaled caches
    vc = rng.integers(0, 256, (nb, bs, HKV, D), dtype=np.uint8) & np.uint8(0xF7)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for window, cap in ((0, 0.0), (3, 0.0), (0, 2.0)):
        out, lse = A.paged_decode_fp8kv(q, kc, vc, (0.3, 0.25), table, cu, bs, 0.2,
                                        window=window, softcap=cap)
        ref_o, ref_l = A.paged_decode(q, 0.3 * dec(kc), 0.25 * dec(vc), table, cu, bs, 0.2,
                                      window=window, softcap=cap)
        assert np.allclose(out, ref_o, rtol=1e-13, atol=1e-13)
        assert np.allclose(lse, ref_l, rtol=1e-13, atol=1e-13)


def _block_lists(rng, blocks, cap, junk=True):
    """Lists (counts [n_qb], indices [n_qb, cap]) holding the True entries of
    the boolean block matrix ``blocks`` [n_qb, n_kb] in shuffled order, with
    junk (out-of-range ids) after each count."""
    n_qb = blocks.shape[0]
    num = np.zeros(n_qb, dtype=np.int32)
    idx = np.full((n_qb, cap), -7 if junk else 0, dtype=np.int32)
    for qb in range(n_qb):
        ids = rng.permutation(np.nonzero(blocks[qb])[0])
        num[qb] = len(ids)
        idx[qb, :len(ids)] = ids
        if junk and len(ids) < cap:
            idx[qb, len(ids):] = rng.choice([-1, blocks.shape[1], 10 ** 6], cap - len(ids))
    return num, idx


def _kron_mask(blocks, q_block, kv_block, q_len, kv_len):
    return np.kron(blocks, np.ones((q_block, kv_block), dtype=bool))[:q_len, :kv_len].astype(bool)


def check_block_visibility_kron(A):
    """No element mask: visibility is the block matrix expanded by np.kron
    (unequal block sizes, ragged edges, shuffled lists, junk past the count)."""
    rng = np.random.default_rng(31)
    q_len, kv_len, qbs, kbs = 23, 37, 3, 5
    n_qb, n_kb = -(-q_len // qbs), -(-kv_len // kbs)
    P = rng.random((n_qb, n_kb)) < 0.4
    F = (rng.random((n_qb, n_kb)) < 0.3) & ~P
    pn, pi = _block_lists(rng, P, n_kb + 2)
    fn, fi = _block_lists(rng, F, n_kb + 2)
    elem = np.ones((q_len, kv_len), dtype=bool)
    got = A.block_visibility(elem, qbs, kbs, pn, pi, fn, fi)
    assert np.array_equal(got, _kron_mask(P | F, qbs, kbs, q_len, kv_len))
    # a count above the capacity reads the whole list and nothing beyond it
    pn2 = pn.copy()
    pn2[0] = 10 ** 6
    got = A.block_visibility(elem, qbs, kbs, pn2, pi, None, None)
    row0 = np.zeros((n_qb, n_kb), dtype=bool)
    row0[0, [k for k in pi[0] if 0 <= k < n_kb]] = True
    exp = _kron_mask(P & (np.arange(n_qb) > 0)[:, None] | row0, qbs, kbs, q_len, kv_len)
    assert np.array_equal(got, exp)


def check_block_all_partial_is_element_mask(A):
    """Every block partial: the element mask alone (causal + window, q shorter
    than kv; document ids)."""
    rng = np.random.default_rng(32)
    q_len, kv_len = 19, 45
    for flags, window, qi, ki in ((ORC.MASK_CAUSAL, 9, None, None),
                                  (ORC.MASK_DOCUMENT, 0, np.sort(rng.integers(0, 3, q_len)),
                                   np.sort(rng.integers(0, 3, kv_len)))):
        elem = A.visibility(q_len, kv_len, flags, qi, ki, window)
        n_qb, n_kb = -(-q_len // 4), -(-kv_len // 8)
        num, idx = _block_lists(rng, np.ones((n_qb, n_kb), dtype=bool), n_kb)
        got = A.block_visibility(elem, 4, 8, num, idx)
        assert np.array_equal(got, elem)


def check_block_causal_lists(A):
    """Causal block lists (diagonal partial, below it full) with a causal
    element mask give np.tril; listing blocks above the diagonal as full
    makes them wholly visible, as partial leaves them hidden."""
    rng = np.random.default_rng(33)
    L, bs = 30, 8
    n = -(-L // bs)
    P = np.eye(n, dtype=bool)
    F = np.tril(np.ones((n, n), dtype=bool), -1)
    pn, pi = _block_lists(rng, P, n)
    fn, fi = _block_lists(rng, F, n)
    elem = A.visibility(L, L, ORC.MASK_CAUSAL)
    assert np.array_equal(A.block_visibility(elem, bs, bs, pn, pi, fn, fi),
                          np.tril(np.ones((L, L), dtype=bool)))
    up = np.triu(np.ones((n, n), dtype=bool), 2)
    fn2, fi2 = _block_lists(rng, F | up, n)
    exp = np.tril(np.ones((L, L), dtype=bool)) | _kron_mask(up, bs, bs, L, L)
    assert np.array_equal(A.block_visibility(elem, bs, bs, pn, pi, fn2, fi2), exp)
    pn3, pi3 = _block_lists(rng, P | up, n)
    assert np.array_equal(A.block_visibility(elem, bs, bs, pn3, pi3, fn, fi),
                          np.tril(np.ones((L, L), dtype=bool)))


def check_block_sparse_attention_vs_sdpa(A):
    """Two sequences, GQA 4/2, causal element mask, a BlockMask with one list
    per mask head (Hm = 1, Hkv, Hq): each head against torch SDPA with the
    explicit mask kron(F) | (kron(P) & tril)."""
    rng = np.random.default_rng(34)
    HQ, HKV, D, qbs, kbs = 4, 2, 8, 4, 8
    lens = [21, 40]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = _rand(rng, cu[-1], HQ, D), _rand(rng, cu[-1], HKV, D), _rand(rng, cu[-1], HKV, D)
    n_qb, n_kb = -(-max(lens) // qbs), -(-max(lens) // kbs)
    for hm in (1, HKV, HQ):
        Ps, Fs = {}, {}
        kv_num = np.zeros((2, hm, n_qb), dtype=np.int32)
        kv_idx = np.zeros((2, hm, n_qb, n_kb), dtype=np.int32)
        full_num, full_idx = np.zeros_like(kv_num), np.zeros_like(kv_idx)
        for b, L in enumerate(lens):
            nq, nk = -(-L // qbs), -(-L // kbs)
            for m in range(hm):
                P = np.zeros((n_qb, n_kb), dtype=bool)
                F = np.zeros((n_qb, n_kb), dtype=bool)
                P[:nq, :nk] = rng.random((nq, nk)) < 0.5
                F[:nq, :nk] = (rng.random((nq, nk)) < 0.3) & ~P[:nq, :nk]
                for qb in range(nq):          # each row keeps its own key
                    kb = (qb * qbs) // kbs
                    if not F[qb, kb]:
                        P[qb, kb] = True
                Ps[b, m], Fs[b, m] = P, F
                kv_num[b, m], kv_idx[b, m] = _block_lists(rng, P, n_kb, junk=False)
                full_num[b, m], full_idx[b, m] = _block_lists(rng, F, n_kb, junk=False)
        bm = A.BlockMask(qbs, kbs, kv_num, kv_idx, full_num, full_idx)
        out, lse = A.attention_varlen(q, k, v, cu, cu, 0.3, ORC.MASK_CAUSAL, block_mask=bm)
        for b, L in enumerate(lens):
            for h in range(HQ):
                m = 0 if hm == 1 else (h if hm == HQ else h // (HQ // HKV))
                mask = (_kron_mask(Fs[b, m], qbs, kbs, L, L)
                        | (_kron_mask(Ps[b, m], qbs, kbs, L, L) & np.tril(np.ones((L, L), dtype=bool))))
                kvh = h // (HQ // HKV)
                ref = _sdpa(q[cu[b]:cu[b + 1], h:h + 1], k[cu[b]:cu[b + 1], kvh:kvh + 1],
                            v[cu[b]:cu[b + 1], kvh:kvh + 1], 0.3, attn_mask=mask)
                assert np.allclose(out[cu[b]:cu[b + 1], h], ref[:, 0], rtol=1e-12, atol=1e-12), (hm, b, h)


def check_unpack_qkv(A):
    row = np.arange(8.0)[None]                       # Hq 2, Hkv 1, D 2
    q, k, v = A.unpack_qkv(row, 2, 1, 2)
    assert np.array_equal(q, [[[0, 1], [2, 3]]])
    assert np.array_equal(k, [[[4, 5]]]) and np.array_equal(v, [[[6, 7]]])
    rng = np.random.default_rng(41)
    x = _rand(rng, 5, (8 + 2 * 2) * 4)
    q, k, v = A.unpack_qkv(x, 8, 2, 4)
    sq, sk, sv = np.split(x, [8 * 4, 10 * 4], axis=1)
    assert np.array_equal(q.reshape(5, -1), sq) and np.array_equal(k.reshape(5, -1), sk)
    assert np.array_equal(v.reshape(5, -1), sv)


def check_new_token_positions(A):
    # a 3-token prefill, a decode step at kv_len 7, a 2-token chunk ending at 5
    got = A.new_token_positions([0, 3, 4, 6], [0, 3, 10, 15])
    assert np.array_equal(got, [0, 1, 2, 6, 3, 4])


def check_rotary_golden(A):
    """A quarter turn (cos 0, sin 1) by hand: non-interleaved pairs (x0, x2),
    (x1, x3); interleaved pairs (x0, x1), (x2, x3); a rotary_dim of 2 leaves
    the last two features alone."""
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    cos, sin = np.zeros((1, 2)), np.ones((1, 2))
    assert np.array_equal(A.rotary(x, [0], cos, sin, 4, False)[0, 0], [-3, -4, 1, 2])
    assert np.array_equal(A.rotary(x, [0], cos, sin, 4, True)[0, 0], [-2, 1, -4, 3])
    assert np.array_equal(A.rotary(x, [0], cos[:, :1], sin[:, :1], 2, False)[0, 0], [-2, 1, 3, 4])
    assert np.array_equal(A.rotary(x, [0], cos, sin, 0, False), x)


def _rope_tables(max_pos, rd, base=10000.0):
    theta = base ** (-np.arange(rd // 2) * 2.0 / rd)
    ang = np.arange(max_pos)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang), ang


def check_rotary_complex_and_permutation(A):
    """Interleaved rotary is the complex product (x_2j + i x_2j+1) e^{i a};
    the non-interleaved one is the interleaved one on features reordered
    (j, j + R/2) -> (2j, 2j + 1)."""
    rng = np.random.default_rng(42)
    T, H, D, R = 6, 3, 12, 8
    cos, sin, ang = _rope_tables(40, R)
    pos = rng.integers(0, 40, T)
    x = _rand(rng, T, H, D)
    got = A.rotary(x, pos, cos, sin, R, True)
    z = (x[..., 0:R:2] + 1j * x[..., 1:R:2]) * np.exp(1j * ang[pos])[:, None, :]
    assert np.allclose(got[..., 0:R:2], z.real, atol=1e-13)
    assert np.allclose(got[..., 1:R:2], z.imag, atol=1e-13)
    assert np.array_equal(got[..., R:], x[..., R:])
    perm = np.empty(R, dtype=int)
    perm[0::2], perm[1::2] = np.arange(R // 2), np.arange(R // 2, R)
    xi = x.copy()
    xi[..., :R] = x[..., perm]
    yi = A.rotary(xi, pos, cos, sin, R, True)
    back = yi.copy()
    back[..., perm] = yi[..., :R]
    assert np.allclose(A.rotary(x, pos, cos, sin, R, False), back, atol=1e-13)


def check_rotary_norm_and_relative_position(A):
    """A rotation keeps each head's norm, and with angle tables p * theta_j
    the product of a rotated q at m and k at n depends on m - n only."""
    rng = np.random.default_rng(43)
    D, R = 16, 16
    cos, sin, _ = _rope_tables(64, R)
    q, k = _rand(rng, 1, 1, D), _rand(rng, 1, 1, D)
    for inter in (False, True):
        y = A.rotary(q, [37], cos, sin, R, inter)
        assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12
        dots = [float(np.sum(A.rotary(q, [m], cos, sin, R, inter)
                             * A.rotary(k, [m - 7], cos, sin, R, inter))) for m in (7, 20, 63)]
        assert np.allclose(dots, dots[0], rtol=0, atol=1e-12)
        plain = float(np.sum(q * k))
        assert abs(dots[0] - plain) > 1e-6          # the angle difference 7 does act


def check_rotary_reshape_and_cache(A):
    """A decode step: the one new token sits at kv_len - 1, its rotated K
    lands in that slot and the rotated Q is returned; V is copied."""
    rng = np.random.default_rng(44)
    H, HKV, D, R, bs = 2, 1, 8, 4, 4
    cos, sin, _ = _rope_tables(16, R)
    q, k, v = _rand(rng, 1, H, D), _rand(rng, 1, HKV, D), _rand(rng, 1, HKV, D)
    kc = np.zeros((4, bs, HKV, D))
    vc = np.zeros((4, bs, HKV, D))
    table = np.array([[2, 0, 3]])
    qr, kc2, vc2 = A.rotary_reshape_and_cache(q, k, v, cos, sin, R, False, kc, vc, table, [0, 1],
                                              [0, 10], bs)
    # position 9: page table[0][2] = 3, slot 1
    assert np.allclose(qr, A.rotary(q, [9], cos, sin, R, False), atol=0)
    assert np.allclose(kc2[3, 1], A.rotary(k, [9], cos, sin, R, False)[0], atol=0)
    assert np.array_equal(vc2[3, 1], v[0])
    assert np.count_nonzero(kc2) == np.count_nonzero(kc2[3, 1])


def _autograd_grads(q, k, v, dout, scale, mask):
    """torch.autograd through CPU fp64 SDPA with an explicit boolean mask;
    q [L, Hq, D], k/v [S, Hkv, D] (GQA by enable_gqa)."""
    Q = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None].requires_grad_()
    K = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None].requires_grad_()
    V = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None].requires_grad_()
    o = F.scaled_dot_product_attention(Q, K, V, attn_mask=torch.from_numpy(mask), scale=scale,
                                       enable_gqa=True)
    o.backward(torch.from_numpy(np.ascontiguousarray(dout.transpose(1, 0, 2)))[None])
    return tuple(t.grad[0].permute(1, 0, 2).numpy() for t in (Q, K, V))


def check_bwd_vs_autograd(A):
    """GQA 4/2, two sequences (one with q shorter than kv), causal and a
    window of 5: the oracle's gradients against autograd through SDPA with
    the mask built from np.tril / np.triu."""
    rng = np.random.default_rng(51)
    HQ, HKV, D = 4, 2, 6
    ql, kl = [9, 5], [9, 12]
    cq, ck = np.concatenate([[0], np.cumsum(ql)]), np.concatenate([[0], np.cumsum(kl)])
    q, k, v = _rand(rng, cq[-1], HQ, D), _rand(rng, ck[-1], HKV, D), _rand(rng, ck[-1], HKV, D)
    do = _rand(rng, cq[-1], HQ, D)
    for window in (0, 5):
        dq, dk, dv = A.attention_varlen_bwd(q, k, v, do, cq, ck, 0.4, ORC.MASK_CAUSAL,
                                            window=window)
        for b in range(2):
            off = kl[b] - ql[b]
            mask = np.tril(np.ones((ql[b], kl[b]), dtype=bool), off)
            if window:
                mask &= np.triu(np.ones((ql[b], kl[b]), dtype=bool), off - window + 1)
            gq, gk, gv = _autograd_grads(q[cq[b]:cq[b + 1]], k[ck[b]:ck[b + 1]],
                                         v[ck[b]:ck[b + 1]], do[cq[b]:cq[b + 1]], 0.4, mask)
            assert np.allclose(dq[cq[b]:cq[b + 1]], gq, rtol=1e-10, atol=1e-12), (window, b)
            assert np.allclose(dk[ck[b]:ck[b + 1]], gk, rtol=1e-10, atol=1e-12), (window, b)
            assert np.allclose(dv[ck[b]:ck[b + 1]], gv, rtol=1e-10, atol=1e-12), (window, b)


def check_bwd_document_and_empty_rows(A):
    """Document ids (non-causal): autograd with the id-equality mask; a
    query whose document has no keys gets dq = 0 and adds nothing to dk, dv."""
    rng = np.random.default_rng(52)
    HQ, HKV, D = 2, 1, 4
    qi = np.array([0, 0, 1, 1, 1, 2, 3], dtype=np.int32)
    ki = np.array([0, 1, 1, 2, 2, 2], dtype=np.int32)
    q, k, v = _rand(rng, 7, HQ, D), _rand(rng, 6, HKV, D), _rand(rng, 6, HKV, D)
    do = _rand(rng, 7, HQ, D)
    dq, dk, dv = A.attention_varlen_bwd(q, k, v, do, [0, 7], [0, 6], 0.7, ORC.MASK_DOCUMENT,
                                        qi, ki)
    assert np.all(dq[6] == 0)                          # document 3 has no keys
    keep = qi != 3
    mask = qi[keep][:, None] == ki[None, :]
    gq, gk, gv = _autograd_grads(q[keep], k, v, do[keep], 0.7, mask)
    assert np.allclose(dq[keep], gq, rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, gk, rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, gv, rtol=1e-10, atol=1e-12)


def check_bwd_finite_differences(A):
    """Central differences of sum(out * dout) on a tiny causal GQA case."""
    rng = np.random.default_rng(53)
    q, k, v = _rand(rng, 3, 2, 2), _rand(rng, 4, 1, 2), _rand(rng, 4, 1, 2)
    do = _rand(rng, 3, 2, 2)
    cq, ck = [0, 3], [0, 4]
    grads = A.attention_varlen_bwd(q, k, v, do, cq, ck, 0.9, ORC.MASK_CAUSAL)

    def loss(q_, k_, v_):
        return float(np.sum(A.attention_varlen(q_, k_, v_, cq, ck, 0.9, ORC.MASK_CAUSAL)[0] * do))

    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(grads[which], num, rtol=1e-6, atol=1e-8), which


def check_bwd_softcap(A):
    """With a score cap: torch.autograd through the composed forward
    (cap * tanh(scale q k^T / cap), masked softmax, P V) in fp64, and central
    differences on a tiny case."""
    rng = np.random.default_rng(54)
    L, S, HQ, HKV, D, cap, scale = 7, 9, 2, 1, 4, 1.5, 0.8
    q, k, v, do = _rand(rng, L, HQ, D), _rand(rng, S, HKV, D), _rand(rng, S, HKV, D), _rand(rng, L, HQ, D)
    q = 2.0 * q                                     # scores large enough for the cap to bend
    dq, dk, dv = A.attention_varlen_bwd(q, k, v, do, [0, L], [0, S], scale, ORC.MASK_CAUSAL,
                                        softcap=cap)
    mask = torch.from_numpy(np.tril(np.ones((L, S), dtype=bool), S - L))
    Q = torch.from_numpy(q).requires_grad_()
    K = torch.from_numpy(k).requires_grad_()
    V = torch.from_numpy(v).requires_grad_()
    outs = []
    for h in range(HQ):
        sc = cap * torch.tanh(scale * (Q[:, h] @ K[:, 0].T) / cap)
        pr = torch.softmax(sc.masked_fill(~mask, float("-inf")), dim=1)
        outs.append(pr @ V[:, 0])
    torch.stack(outs, dim=1).backward(torch.from_numpy(do))
    assert np.allclose(dq, Q.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, K.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, V.grad.numpy(), rtol=1e-10, atol=1e-12)
    # central differences on a smaller case
    q2, k2, v2, do2 = q[:3, :1, :2], k[:4, :, :2], v[:4, :, :2], do[:3, :1, :2]
    g = A.attention_varlen_bwd(q2, k2, v2, do2, [0, 3], [0, 4], 0.9, ORC.MASK_CAUSAL, softcap=0.7)

    def loss(a, b, c):
        o = A.attention_varlen(a, b, c, [0, 3], [0, 4], 0.9, ORC.MASK_CAUSAL, softcap=0.7)[0]
        return float(np.sum(o * do2))

    eps = 1e-6
    for which, x in enumerate((q2, k2, v2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = [q2, k2, v2], [q2, k2, v2]
            ap[which], am[which] = xp, xm
            num[idx] = (loss(*ap) - loss(*am)) / (2 * eps)
        assert np.allclose(g[which], num, rtol=1e-6, atol=1e-8), which


def check_window_bands(A):
    """Causal + window W: a band of W keys ending on the (bottom-right) diagonal,
    built here from np.tril / np.triu; without CAUSAL the window only bounds j
    from below; a window wider than the sequence changes nothing."""
    for q_len, kv_len, W in ((7, 7, 1), (7, 7, 3), (5, 9, 2), (9, 5, 4), (6, 6, 100)):
        off = kv_len - q_len
        ones = np.ones((q_len, kv_len), bool)
        band = np.tril(ones, k=off) & np.triu(ones, k=off - W + 1)
        assert np.array_equal(A.visibility(q_len, kv_len, ORC.MASK_CAUSAL, window=W), band)
    assert np.array_equal(A.visibility(4, 6, 0, window=2), np.triu(np.ones((4, 6), bool), k=1))
    assert np.array_equal(A.visibility(6, 6, ORC.MASK_CAUSAL, window=6),
                          A.visibility(6, 6, ORC.MASK_CAUSAL))


def check_window_vs_sdpa(A):
    """Causal + window against torch SDPA given the same band as an explicit mask."""
    rng = np.random.default_rng(8)
    L, H, D, W = 19, 2, 8, 5
    q, k, v = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    ones = np.ones((L, L), bool)
    band = np.tril(ones) & np.triu(ones, k=-(W - 1))
    out, _ = A.attention_varlen(q, k, v, [0, L], [0, L], 0.41, ORC.MASK_CAUSAL, window=W)
    ref = _sdpa(q, k, v, 0.41, attn_mask=band)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def check_window_one_is_diagonal(A):
    """Window 1 with causal leaves each row its own (bottom-right) key: O is that
    V row exactly and LSE is its scaled score."""
    rng = np.random.default_rng(9)
    q_len, kv_len, D = 5, 8, 6
    q, k, v = _rand(rng, q_len, 1, D), _rand(rng, kv_len, 1, D), _rand(rng, kv_len, 1, D)
    out, lse = A.attention_varlen(q, k, v, [0, q_len], [0, kv_len], 0.3, ORC.MASK_CAUSAL, window=1)
    for i in range(q_len):
        j = i + kv_len - q_len
        assert np.array_equal(out[i, 0], v[j, 0])
        assert abs(lse[i, 0] - 0.3 * float(q[i, 0] @ k[j, 0])) < 1e-12


def check_window_decode_is_truncated_cache(A):
    """Decode with window W equals decode without one over the last W keys only
    (through the paged path with an identity block table)."""
    rng = np.random.default_rng(10)
    lens, bs, W, Hq, Hkv, D = [13, 4, 9], 4, 6, 4, 2, 8
    q = _rand(rng, len(lens), Hq, D)
    out, lse = None, None
    ks = [_rand(rng, n, Hkv, D) for n in lens]
    vs = [_rand(rng, n, Hkv, D) for n in lens]
    def paged(parts):
        nbs = [(p.shape[0] + bs - 1) // bs for p in parts]
        cache = np.zeros((sum(nbs), bs, Hkv, D))
        table = np.zeros((len(parts), max(nbs)), dtype=np.int32)
        blk = 0
        for b, p in enumerate(parts):
            for j in range(p.shape[0]):
                cache[blk + j // bs, j % bs] = p[j]
            table[b, :nbs[b]] = np.arange(blk, blk + nbs[b])
            blk += nbs[b]
        return cache, table
    kc, table = paged(ks)
    vc, _ = paged(vs)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, lse = A.paged_decode(q, kc, vc, table, cu, bs, 0.35, window=W)
    cut = [min(W, n) for n in lens]
    kc2, table2 = paged([p[-c:] for p, c in zip(ks, cut)])
    vc2, _ = paged([p[-c:] for p, c in zip(vs, cut)])
    out2, lse2 = A.paged_decode(q, kc2, vc2, table2, np.concatenate([[0], np.cumsum(cut)]), bs, 0.35)
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def check_softcap_saturated(A):
    """A huge scale drives every capped score to +-c (c = 50, the softcap value
    in [ORT] Testing): keys with q.k > 0 weigh e^c, the others e^-c."""
    rng = np.random.default_rng(11)
    n, D, c = 9, 8, 50.0
    q = _rand(rng, 1, 1, D)
    k = _rand(rng, n, 1, D)
    dots = k[:, 0] @ q[0, 0]
    k[np.abs(dots) < 0.1] *= 0.0
    k[np.abs(dots) < 0.1, 0, 0] = 1.0 / q[0, 0, 0]       # q.k = 1 for those rows
    dots = k[:, 0] @ q[0, 0]
    v = _rand(rng, n, 1, D)
    out, lse = A.attention_varlen(q, k, v, [0, 1], [0, n], 1e6, softcap=c)
    sign = np.where(dots > 0, 1.0, -1.0)
    w = np.exp(sign * c - c)                               # shifted by the max, c
    assert np.allclose(out[0, 0], (w @ v[:, 0]) / w.sum(), rtol=1e-12, atol=1e-12)
    assert abs(lse[0, 0] - (c + math.log(w.sum()))) < 1e-12


def check_softcap_large_cap_limit(A):
    """c -> infinity recovers the uncapped scores; a finite cap keeps every
    score in [-c, c] (tanh saturates to exactly +-1 in fp64 for large
    arguments), so LSE lies within c of ln(visible keys)."""
    rng = np.random.default_rng(12)
    L, H, D = 11, 2, 8
    q, k, v = _rand(rng, L, H, D), _rand(rng, L, H, D), _rand(rng, L, H, D)
    o0, l0 = A.attention_varlen(q, k, v, [0, L], [0, L], 0.5, ORC.MASK_CAUSAL)
    o1, l1 = A.attention_varlen(q, k, v, [0, L], [0, L], 0.5, ORC.MASK_CAUSAL, softcap=1e7)
    assert np.allclose(o0, o1, rtol=1e-9, atol=1e-9) and np.allclose(l0, l1, rtol=1e-9, atol=1e-9)
    c = 0.25
    _, l2 = A.attention_varlen(q, k, v, [0, L], [0, L], 40.0, ORC.MASK_CAUSAL, softcap=c)
    n = np.arange(1, L + 1)[:, None]
    assert np.all(l2 <= np.log(n) + c + 1e-12) and np.all(l2 >= np.log(n) - c - 1e-12)
    assert np.ptp(l2 - np.log(n)) > 0.1      # the cap is not a constant shift


CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__[len("check_"):])
def test_oracle_pin(check):
    check(ORC)


def test_pin_status_covers_exports():
    import oracle
    for name in ("cu_seqlens", "reshape_and_cache", "gather_paged", "visibility",
                 "attention_varlen", "paged_attention", "paged_decode", "e4m3_decode",
                 "fp8_attention", "default_scale", "paged_decode_fp8kv", "block_visibility", "unpack_qkv",
                 "new_token_positions", "rotary", "rotary_reshape_and_cache",
                 "attention_varlen_bwd"):
        assert hasattr(oracle, name)
        assert "pinned" in ORC.PIN_STATUS[name]


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one check fail
# ----------------------------------------------------------------------------

def _mut_visibility_off_by_one(orig):
    def f(q_len, kv_len, flags, q_ids=None, kv_ids=None, window=0):
        vis = orig(q_len, kv_len, flags & ~ORC.MASK_CAUSAL, q_ids, kv_ids, window)
        if flags & ORC.MASK_CAUSAL:
            i = np.arange(q_len)[:, None]
            j = np.arange(kv_len)[None, :]
            vis &= j < i + (kv_len - q_len)
        return vis
    return f


def _mut_visibility_top_left(orig):
    def f(q_len, kv_len, flags, q_ids=None, kv_ids=None, window=0):
        vis = orig(q_len, kv_len, flags & ~ORC.MASK_CAUSAL, q_ids, kv_ids, window)
        if flags & ORC.MASK_CAUSAL:
            vis &= np.arange(kv_len)[None, :] <= np.arange(q_len)[:, None]
        return vis
    return f


def _mut_visibility_patch_strict(orig):
    def f(q_len, kv_len, flags, q_ids=None, kv_ids=None, window=0):
        vis = orig(q_len, kv_len, flags, q_ids, kv_ids, window)
        if flags & ORC.MASK_PATCH:
            vis &= np.arange(kv_len)[None, :] < np.asarray(q_ids)[:q_len, None]
        return vis
    return f


def _mut_attention_scale_dropped(orig):
    def f(q, k, v, cu_q, cu_kv, scale, *a, **kw):
        return orig(q, k, v, cu_q, cu_kv, 1.0, *a, **kw)
    return f


def _mut_attention_gqa_modulo(orig):
    # q head h reads kv head h % Hkv instead of h // G: permute the q heads going in and out
    def f(q, k, v, cu_q, cu_kv, scale, *a, **kw):
        q = np.asarray(q, dtype=np.float64)
        hq, hkv = q.shape[1], np.asarray(k).shape[1]
        g = hq // hkv
        perm = np.array([(h % hkv) * g + h // hkv for h in range(hq)])
        out, lse = orig(q[:, perm], k, v, cu_q, cu_kv, scale, *a, **kw)
        inv = np.argsort(perm)
        return out[:, inv], lse[:, inv]
    return f


def _mut_softmax_no_normalise(orig):
    def f(s, vis, v):
        out, lse = orig(s, vis, v)
        counts = vis.sum(axis=1)
        return out * np.maximum(counts, 1)[:, None], lse
    return f


def _mut_softmax_log2_lse(orig):
    def f(s, vis, v):
        out, lse = orig(s, vis, v)
        return out, lse / math.log(2.0)
    return f


def _mut_softmax_kv_swapped(orig):
    def f(s, vis, v):
        return orig(s.T[:s.shape[0]] if s.shape[0] == s.shape[1] else s * 0.5, vis, v)
    return f


def _mut_gather_slot_reversed(orig):
    def f(cache, table_row, kv_len, block_size):
        out = np.empty((kv_len,) + tuple(cache.shape[2:]), dtype=cache.dtype)
        for j in range(kv_len):
            out[j] = cache[int(table_row[j // block_size]), block_size - 1 - j % block_size]
        return out
    return f


def _mut_reshape_from_start(orig):
    def f(k_new, v_new, k_cache, v_cache, table, cu_new, cu_kv, bs):
        return orig(k_new, v_new, k_cache, v_cache, table, cu_new, cu_new, bs)
    return f


def _mut_e4m3_bias8(orig):
    def f(codes):
        return orig(codes) * 0.5
    return f


def _mut_cu_inclusive(orig):
    def f(lens):
        out = orig(lens)
        return np.concatenate([out[1:], out[-1:]]).astype(np.int32)
    return f


def _mut_fp8_v_rowmajor(orig):
    def f(q8, k8, v8, descale, *a, **kw):
        h, d, t = v8.shape
        return orig(q8, k8, np.ascontiguousarray(v8).reshape(h, t, d).transpose(0, 2, 1), descale,
                    *a, **kw)
    return f


def _mut_default_scale_inverse(orig):
    return lambda e: math.sqrt(e)


def _mut_window_one_extra_key(orig):
    def f(q_len, kv_len, flags, q_ids=None, kv_ids=None, window=0):
        return orig(q_len, kv_len, flags, q_ids, kv_ids, window + 1 if window > 0 else 0)
    return f


def _mut_window_top_left(orig):
    def f(q_len, kv_len, flags, q_ids=None, kv_ids=None, window=0):
        vis = orig(q_len, kv_len, flags, q_ids, kv_ids, 0)
        if window > 0:
            vis &= np.arange(kv_len)[None, :] > np.arange(q_len)[:, None] - window
        return vis
    return f


def _mut_softcap_no_division(orig):
    # c * tanh(s) instead of c * tanh(s / c): scale the cap into the scores
    def f(q, k, v, cu_q, cu_kv, scale, *a, softcap=0.0, **kw):
        if softcap <= 0:
            return orig(q, k, v, cu_q, cu_kv, scale, *a, **kw)
        return orig(q, k, v, cu_q, cu_kv, scale * softcap, *a, softcap=softcap * softcap, **kw)
    return f


def _mut_fp8kv_descales_swapped(orig):
    def f(q, k8, v8, kv_descale, *a, **kw):
        return orig(q, k8, v8, tuple(kv_descale)[::-1], *a, **kw)
    return f


def _mut_block_full_masked(orig):
    # full blocks treated like partial ones (element mask evaluated there too)
    def f(elem_vis, q_block, kv_block, kv_num, kv_idx, full_num=None, full_idx=None):
        out = orig(elem_vis, q_block, kv_block, kv_num, kv_idx, full_num, full_idx)
        return out & elem_vis
    return f


def _mut_block_index_shift(orig):
    def f(elem_vis, q_block, kv_block, kv_num, kv_idx, full_num=None, full_idx=None):
        sh = lambda x: None if x is None else np.asarray(x) + 1
        return orig(elem_vis, q_block, kv_block, kv_num, sh(kv_idx), full_num, sh(full_idx))
    return f


def _mut_block_sizes_swapped(orig):
    def f(elem_vis, q_block, kv_block, *a, **kw):
        return orig(elem_vis, kv_block, q_block, *a, **kw)
    return f


def _mut_mask_head_modulo(orig):
    def f(h, hq, hkv, hm):
        if hm == hkv and hm != hq and hm != 1:
            return h % hkv
        return orig(h, hq, hkv, hm)
    return f


def _mut_rotary_sin_sign(orig):
    def f(x, positions, cos_table, sin_table, rotary_dim, interleaved):
        return orig(x, positions, cos_table, -np.asarray(sin_table), rotary_dim, interleaved)
    return f


def _mut_rotary_pairing(orig):
    def f(x, positions, cos_table, sin_table, rotary_dim, interleaved):
        return orig(x, positions, cos_table, sin_table, rotary_dim, not interleaved)
    return f


def _mut_positions_from_zero(orig):
    def f(cu_new, cu_kv):
        return orig(cu_new, cu_new)
    return f


def _mut_unpack_kv_swapped(orig):
    def f(qkv, hq, hkv, d):
        q, k, v = orig(qkv, hq, hkv, d)
        return q, v, k
    return f


def _bwd_variant(drop_delta=False, no_gqa_sum=False):
    """The oracle's backward with one planted mistake (same steps otherwise)."""
    def f(q, k, v, dout, cu_q, cu_kv, scale, flags=0, q_ids=None, kv_ids=None, window=0,
          softcap=0.0):
        q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        hq, hkv = q.shape[1], k.shape[1]
        g = hq // hkv
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(len(cu_q) - 1):
            q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_kv[b]), int(cu_kv[b + 1])
            qi = None if q_ids is None else np.asarray(q_ids)[q0:q1]
            ki = None if kv_ids is None else np.asarray(kv_ids)[k0:k1]
            vis = ORC.visibility(q1 - q0, k1 - k0, flags, qi, ki, window)
            for h in range(hq):
                kvh = h // g
                Q, K, V, dO = q[q0:q1, h], k[k0:k1, kvh], v[k0:k1, kvh], dout[q0:q1, h]
                raw = scale * (Q @ K.T)
                if softcap > 0:
                    th = np.tanh(raw / softcap)
                    raw = softcap * th
                s_ = np.where(vis, raw, -np.inf)
                m = s_.max(axis=1, initial=-np.inf, keepdims=True)
                e = np.where(vis, np.exp(s_ - np.where(np.isfinite(m), m, 0.0)), 0.0)
                tot = e.sum(axis=1, keepdims=True)
                P = np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)
                dP = dO @ V.T
                dS = P * dP if drop_delta else P * (dP - (dP * P).sum(axis=1, keepdims=True))
                if softcap > 0:
                    dS = dS * (1.0 - th * th)
                if no_gqa_sum:
                    dv[k0:k1, kvh] = P.T @ dO
                    dk[k0:k1, kvh] = scale * (dS.T @ Q)
                else:
                    dv[k0:k1, kvh] += P.T @ dO
                    dk[k0:k1, kvh] += scale * (dS.T @ Q)
                dq[q0:q1, h] = scale * (dS @ K)
        return dq, dk, dv
    return f


def _mut_bwd_drop_delta(orig):
    return _bwd_variant(drop_delta=True)


def _mut_bwd_no_gqa_sum(orig):
    return _bwd_variant(no_gqa_sum=True)


def _mut_bwd_dq_unscaled(orig):
    def f(q, k, v, dout, cu_q, cu_kv, scale, *a, **kw):
        dq, dk, dv = orig(q, k, v, dout, cu_q, cu_kv, scale, *a, **kw)
        return dq / scale, dk, dv
    return f


def _mut_bwd_cap_derivative_dropped(orig):
    # gradient of the uncapped scores reported for a capped forward
    def f(q, k, v, dout, cu_q, cu_kv, scale, flags=0, q_ids=None, kv_ids=None, window=0,
          softcap=0.0):
        if softcap <= 0:
            return orig(q, k, v, dout, cu_q, cu_kv, scale, flags, q_ids, kv_ids, window)
        return orig(q, k, v, dout, cu_q, cu_kv, scale, flags, q_ids, kv_ids, window, 1e12)
    return f


MUTATIONS = {
    "causal_off_by_one": ("visibility", _mut_visibility_off_by_one),
    "causal_top_left": ("visibility", _mut_visibility_top_left),
    "patch_strict": ("visibility", _mut_visibility_patch_strict),
    "scale_dropped": ("attention_varlen", _mut_attention_scale_dropped),
    "gqa_modulo_map": ("attention_varlen", _mut_attention_gqa_modulo),
    "no_normalisation": ("_softmax_rows", _mut_softmax_no_normalise),
    "lse_in_log2": ("_softmax_rows", _mut_softmax_log2_lse),
    "scores_perturbed": ("_softmax_rows", _mut_softmax_kv_swapped),
    "gather_slot_reversed": ("gather_paged", _mut_gather_slot_reversed),
    "reshape_positions_from_start": ("reshape_and_cache", _mut_reshape_from_start),
    "e4m3_wrong_bias": ("e4m3_decode", _mut_e4m3_bias8),
    "cu_seqlens_inclusive": ("cu_seqlens", _mut_cu_inclusive),
    "fp8_v_read_row_major": ("fp8_attention", _mut_fp8_v_rowmajor),
    "default_scale_inverted": ("default_scale", _mut_default_scale_inverse),
    "window_one_extra_key": ("visibility", _mut_window_one_extra_key),
    "window_top_left": ("visibility", _mut_window_top_left),
    "softcap_no_division": ("attention_varlen", _mut_softcap_no_division),
    "fp8kv_descales_swapped": ("paged_decode_fp8kv", _mut_fp8kv_descales_swapped),
    "block_full_masked": ("block_visibility", _mut_block_full_masked),
    "block_index_shift": ("block_visibility", _mut_block_index_shift),
    "block_sizes_swapped": ("block_visibility", _mut_block_sizes_swapped),
    "block_mask_head_modulo": ("_mask_head", _mut_mask_head_modulo),
    "rotary_sin_sign": ("rotary", _mut_rotary_sin_sign),
    "rotary_pairing_swapped": ("rotary", _mut_rotary_pairing),
    "positions_from_zero": ("new_token_positions", _mut_positions_from_zero),
    "unpack_kv_swapped": ("unpack_qkv", _mut_unpack_kv_swapped),
    "bwd_drop_delta": ("attention_varlen_bwd", _mut_bwd_drop_delta),
    "bwd_no_gqa_sum": ("attention_varlen_bwd", _mut_bwd_no_gqa_sum),
    "bwd_dq_unscaled": ("attention_varlen_bwd", _mut_bwd_dq_unscaled),
    "bwd_cap_derivative_dropped": ("attention_varlen_bwd", _mut_bwd_cap_derivative_dropped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(name, monkeypatch):
    attr, make = MUTATIONS[name]
    monkeypatch.setattr(ORC, attr, make(getattr(ORC, attr)))
    caught = []
    for check in CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(ORC)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"planted mistake {name} passed every pin"
