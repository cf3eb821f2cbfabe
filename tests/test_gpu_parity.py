"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: integer / byte / index work bit-exact; fp16 and bf16 outputs within
max-abs 2e-2 and relative L2 1e-2; fp8 within max-abs 6e-2; LSE within 2e-3.
Sizes are small enough for the oracle to finish in seconds but span several
query and key tiles with ragged tails.
"""

import math

import numpy as np
import pytest
import torch

import oracle as ORC
import workloads as W
from gpu_common import (ATOL_16, ATOL_FP8, DEV, LSE_ATOL_FP8, REL_16, banner, compare, gpu_cache, gpu_decode,
                        gpu_fp8, gpu_prefill, lib_module, oracle_decode, oracle_fp8,
                        oracle_prefill, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def A():
    return lib_module()


# ------------------------------------------------------------------ a1, a2

@pytest.mark.parametrize("n", [1, 2, 16, 64, 1000, 1025, 3000])
def test_cu_seqlens_bit_exact(A, n):
    banner(f"cu_seqlens n={n}")
    rng = np.random.default_rng(n)
    lens = rng.integers(0, 5000, n).astype(np.int32)
    lens[rng.integers(0, n, max(1, n // 7))] = 0
    got = A.attn_cu_seqlens(torch.from_numpy(lens).to(DEV)).cpu().numpy()
    assert np.array_equal(got, ORC.cu_seqlens(lens))


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.uint8).cpu().numpy()


@pytest.mark.parametrize("dtype,hkv,d,bs", [("bf16", 8, 128, 16), ("f16", 2, 64, 32),
                                             ("bf16", 1, 64, 64), ("fp8", 4, 128, 16)])
def test_reshape_and_cache_bit_exact(A, dtype, hkv, d, bs):
    """Two appends (a prefix, then a few new tokens per sequence) into a
    NaN-poisoned pool; every cache byte must match the oracle's scatter."""
    banner(f"reshape_and_cache {dtype} hkv={hkv} d={d} bs={bs}")
    rng = np.random.default_rng(7)
    kv_lens = np.array([1, 40, 0, 129, 17], dtype=np.int32)
    pre_lens = np.array([0, 33, 0, 100, 16], dtype=np.int32)
    tail = kv_lens - pre_lens
    table, nb = W._block_table(rng, kv_lens, bs)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.uint8}[dtype]
    shape = (nb, bs, hkv, d)

    def toks(n):
        x = torch.randn((int(n), hkv, d), generator=torch.Generator().manual_seed(int(n) + 1))
        return x.to(tdt) if dtype != "fp8" else (x * 40).to(torch.float8_e4m3fn).view(torch.uint8)

    k1, v1, k2, v2 = toks(pre_lens.sum()), toks(pre_lens.sum()), toks(tail.sum()), toks(tail.sum())
    poison = torch.full(shape, float("nan")).to(tdt) if dtype != "fp8" else \
        torch.full(shape, 0x7F, dtype=torch.uint8)
    kc, vc = poison.clone().to(DEV), poison.clone().to(DEV)
    bt = torch.from_numpy(table).to(DEV)
    cu_pre = A.attn_cu_seqlens(torch.from_numpy(pre_lens).to(DEV))
    cu_tail = A.attn_cu_seqlens(torch.from_numpy(tail).to(DEV))
    cu_kv = A.attn_cu_seqlens(torch.from_numpy(kv_lens).to(DEV))
    A.attn_reshape_and_cache(k1.to(DEV), v1.to(DEV), kc, vc, bt, cu_pre, cu_pre)
    A.attn_reshape_and_cache(k2.to(DEV), v2.to(DEV), kc, vc, bt, cu_tail, cu_kv)
    torch.cuda.synchronize()

    rk, rv = _bits(poison), _bits(poison)
    rk, rv = ORC.reshape_and_cache(_bits(k1), _bits(v1), rk, rv, table, ORC.cu_seqlens(pre_lens),
                                   ORC.cu_seqlens(pre_lens), bs)
    rk, rv = ORC.reshape_and_cache(_bits(k2), _bits(v2), rk, rv, table, ORC.cu_seqlens(tail),
                                   ORC.cu_seqlens(kv_lens), bs)
    assert np.array_equal(_bits(kc), rk)
    assert np.array_equal(_bits(vc), rv)


# ------------------------------------------------------------------ prefill

def _check_prefill(A, w, what):
    banner(f"prefill {what} B={w.batch} q={w.q_lens.tolist()[:6]} kv={w.kv_lens.tolist()[:6]} "
           f"H={w.num_heads}/{w.num_kv_heads} D={w.head_size} bs={w.block_size} mask={w.mask_flags}")
    out, lse = gpu_prefill(w, A)
    ref_o, ref_l = oracle_prefill(w)
    return compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=what)


def test_prefill_tiny_gqa_causal_fp16(A):
    _check_prefill(A, W.tiny_gqa_causal_fp16(), "tiny_gqa_causal_fp16")


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 128), (16, 2, 64), (4, 4, 64),
                                      (12, 3, 128)])
def test_prefill_varlen_causal_bf16(A, hq, hkv, d):
    lens = [300, 77, 1, 513, 64]
    w = W.make_prefill("varlen", 11, "bf16", lens, lens, hq, hkv, d, 16, W.MASK_CAUSAL)
    _check_prefill(A, w, f"varlen_causal_bf16_{hq}x{hkv}_d{d}")


@pytest.mark.parametrize("bs", [32, 64])
def test_prefill_block_sizes(A, bs):
    lens = [200, 97]
    w = W.make_prefill("bs", 12, "bf16", lens, lens, 8, 2, 128, bs, W.MASK_CAUSAL)
    _check_prefill(A, w, f"block_size_{bs}")


def test_prefill_no_mask_cross_lengths(A):
    w = W.make_prefill("nomask", 13, "f16", [5, 130, 260], [300, 7, 260], 4, 2, 128, 16,
                       W.MASK_NONE)
    _check_prefill(A, w, "no_mask_q_ne_kv")


def test_prefill_causal_bottom_right(A):
    """Chunked prefill: q_len < kv_len, the queries are the last tokens."""
    w = W.make_prefill("chunk", 14, "bf16", [50, 130, 1], [400, 131, 77], 8, 2, 128, 16,
                       W.MASK_CAUSAL)
    _check_prefill(A, w, "causal_bottom_right")


def test_prefill_fully_masked_rows(A):
    """kv_len = 0, and causal with q_len > kv_len: rows with no key give 0 / -inf."""
    w = W.make_prefill("masked", 15, "bf16", [40, 70, 9], [0, 30, 9], 4, 1, 64, 16,
                       W.MASK_CAUSAL)
    st = _check_prefill(A, w, "fully_masked_rows")


def test_prefill_byte_patch_cross_small(A):
    w = W.byte_patch_cross_bf16(batch=2, n_bytes=700, n_keys=96, seed=21)
    _check_prefill(A, w, "byte_patch_cross_small")


def test_prefill_document_mask(A):
    rng = np.random.default_rng(5)
    lens = [260, 190]
    docs = []
    for n in lens:
        cuts = np.sort(rng.choice(np.arange(1, n), 4, replace=False))
        docs.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
    ids = np.concatenate(docs)
    for flags in (W.MASK_DOCUMENT, W.MASK_DOCUMENT | W.MASK_CAUSAL):
        w = W.make_prefill("doc", 16, "bf16", lens, lens, 8, 4, 64, 16, flags, q_ids=ids,
                           kv_ids=ids)
        _check_prefill(A, w, f"document_mask_{flags}")


def test_prefill_visibility_probe_bit_exact(A):
    """scale = 0 makes every visible key weigh the same, and V_j = onehot(j mod D)
    turns O_i * n_i into per-residue counts of row i's visible keys: the visible
    set sizes recovered from the GPU output must equal the oracle's exactly."""
    lens_q, lens_kv = [70, 33], [90, 33]
    D = 64
    w = W.make_prefill("probe", 17, "bf16", lens_q, lens_kv, 4, 2, D, 16, W.MASK_CAUSAL)
    tk = w.total_kv
    onehot = torch.zeros((tk, 2, D))
    cu = np.concatenate([[0], np.cumsum(lens_kv)])
    for b in range(2):
        for j in range(lens_kv[b]):
            onehot[cu[b] + j, :, j % D] = 1.0
    w.v_new = onehot.to(torch.bfloat16)
    out, lse = gpu_prefill(w, A, scale=0.0)
    o = out.float().cpu().numpy()
    cuq = np.concatenate([[0], np.cumsum(lens_q)])
    for b in range(2):
        vis = ORC.visibility(lens_q[b], lens_kv[b], ORC.MASK_CAUSAL)
        for i in range(lens_q[b]):
            n = int(vis[i].sum())
            res = np.bincount(np.nonzero(vis[i])[0] % D, minlength=D)
            for h in range(4):
                got = o[cuq[b] + i, h]
                assert np.array_equal(np.rint(got * n), res), (b, i, h)
                assert abs(float(lse[cuq[b] + i, h]) - math.log(n)) < 1e-5


def test_prefill_single_key_rows_exact(A):
    """Causal row 0 of each sequence sees only key 0: O = V[0] exactly."""
    lens = [45, 300, 17]
    w = W.make_prefill("single", 18, "bf16", lens, lens, 8, 2, 128, 16, W.MASK_CAUSAL)
    out, _ = gpu_prefill(w, A)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for b in range(3):
        for h in range(8):
            assert torch.equal(out[cu[b], h].cpu(), w.v_new[cu[b], h // 4])


def test_prefill_block_table_permutation_bitwise(A):
    """The same tokens placed in two different page orders give identical bits."""
    lens = [300, 150]
    w = W.make_prefill("perm", 19, "bf16", lens, lens, 8, 2, 128, 16, W.MASK_CAUSAL)
    out1, lse1 = gpu_prefill(w, A)
    rng = np.random.default_rng(99)
    w2 = W.make_prefill("perm", 19, "bf16", lens, lens, 8, 2, 128, 16, W.MASK_CAUSAL, rng=rng)
    assert not np.array_equal(w.block_table, w2.block_table)
    out2, lse2 = gpu_prefill(w2, A)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_prefill_sequence_alone_equals_in_batch(A):
    lens = [300, 150, 200]
    w = W.make_prefill("batch", 20, "bf16", lens, lens, 8, 2, 128, 16, W.MASK_CAUSAL)
    out, lse = gpu_prefill(w, A)
    w1 = W.make_prefill("alone", 20, "bf16", [150], [150], 8, 2, 128, 16, W.MASK_CAUSAL)
    w1.q = w.q[300:450].clone()
    w1.k_new = w.k_new[300:450].clone()
    w1.v_new = w.v_new[300:450].clone()
    out1, lse1 = gpu_prefill(w1, A)
    assert torch.equal(out[300:450], out1) and torch.equal(lse[300:450], lse1)


# ------------------------------------------------------------------ decode

def test_decode_small_and_split_invariance(A):
    w = W.make_decode("dec", 31, "bf16", [1, 17, 300, 1000, 2500, 0, 4096], 32, 8, 128, 16)
    banner("decode small")
    cache = gpu_cache(w, A)
    ref_o, ref_l = oracle_decode(w)
    outs = []
    for st in (0, 256, 512, 1024):
        out, lse = gpu_decode(w, A, split_tokens=st, cache=cache)
        compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"decode split={st}")
        outs.append(out.float())
    for o in outs[1:]:
        assert torch.allclose(o, outs[0], rtol=1e-2, atol=1e-2)
    again, _ = gpu_decode(w, A, split_tokens=256, cache=cache)
    assert torch.equal(again.float(), outs[1])


def test_decode_d64_fp16(A):
    w = W.make_decode("dec64", 32, "f16", [33, 700, 129], 16, 2, 64, 32)
    banner("decode d64 fp16")
    out, lse = gpu_decode(w, A)
    ref_o, ref_l = oracle_decode(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="decode_d64_fp16")


def test_decode_equals_last_prefill_row(A):
    lens = [90, 513, 260]
    w = W.make_prefill("lastrow", 33, "bf16", lens, lens, 32, 8, 128, 16, W.MASK_CAUSAL)
    cache = gpu_cache(w, A)
    out_p, _ = gpu_prefill(w, A, cache=cache)
    cu = np.concatenate([[0], np.cumsum(lens)])
    last = torch.as_tensor(cu[1:] - 1)
    wd = W.make_decode("lastrow", 33, "bf16", lens, 32, 8, 128, 16)
    wd.q = w.q[last].contiguous()
    kc, vc, bt, cu_kv = cache
    out_d, _ = A.attn_paged_decode_fwd(wd.q.to(DEV), kc, vc, bt, cu_kv, max(lens),
                                       return_lse=True)
    torch.cuda.synchronize()
    assert torch.allclose(out_d.float(), out_p[last.to(DEV)].float(), atol=1e-2, rtol=1e-2)


# ------------------------------------------------------------------ fp8

@pytest.mark.parametrize("lens,hq,hkv", [([300, 200], 4, 4), ([129, 64, 257], 8, 2)])
def test_fp8_causal(A, lens, hq, hkv):
    w = W.make_fp8("fp8", 41, lens, lens, hq, hkv, 128, W.MASK_CAUSAL)
    banner(f"fp8 causal lens={lens} H={hq}/{hkv}")
    out, lse = gpu_fp8(w, A)
    ref_o, ref_l = oracle_fp8(w)
    compare(out, lse, ref_o, ref_l, ATOL_FP8, what=f"fp8_causal_{lens}", lse_atol=LSE_ATOL_FP8)


@pytest.mark.parametrize("q_lens,kv_lens,hq,hkv", [
    ([1024, 640], [1024, 640], 16, 2),    # many tiles through the ring, V^T aligned
    ([1000, 777], [1000, 777], 4, 4),     # many tiles, V^T unaligned (total 1777)
    ([40, 600], [40, 600], 8, 8),         # total aligned, second sequence starts at key 40
    ([100, 37], [700, 301], 8, 2),        # bottom-right causal, q shorter than kv
])
def test_fp8_causal_multi_tile(A, q_lens, kv_lens, hq, hkv):
    w = W.make_fp8("fp8m", 43, q_lens, kv_lens, hq, hkv, 128, W.MASK_CAUSAL)
    banner(f"fp8 causal q={q_lens} kv={kv_lens} H={hq}/{hkv}")
    out, lse = gpu_fp8(w, A)
    ref_o, ref_l = oracle_fp8(w)
    compare(out, lse, ref_o, ref_l, ATOL_FP8, what=f"fp8_multi_{q_lens}_{kv_lens}",
            lse_atol=LSE_ATOL_FP8)


def test_fp8_document_mask_negative_scale(A):
    """Document ids bound each row's keys on both sides; a negative scale
    flips the sign of every score."""
    rng = np.random.default_rng(7)
    lens = [530, 333]
    docs = []
    for n in lens:
        cuts = np.sort(rng.choice(np.arange(1, n), 5, replace=False))
        docs.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
    ids = np.concatenate(docs)
    for flags, scale in ((W.MASK_DOCUMENT, -0.07), (W.MASK_DOCUMENT | W.MASK_CAUSAL, 0.09)):
        w = W.make_fp8("fp8doc", 44, lens, lens, 8, 2, 128, flags, q_ids=ids, kv_ids=ids,
                       scale=scale)
        banner(f"fp8 document flags={flags} scale={scale}")
        out, lse = gpu_fp8(w, A)
        ref_o, ref_l = oracle_fp8(w)
        compare(out, lse, ref_o, ref_l, ATOL_FP8, what=f"fp8_document_{flags}",
                lse_atol=LSE_ATOL_FP8)


def test_fp8_unaligned_varlen_no_mask(A):
    """Lengths that are not multiples of 16 exercise the unaligned V path."""
    w = W.make_fp8("fp8u", 42, [37, 100, 5], [50, 77, 130], 4, 2, 128, W.MASK_NONE)
    banner("fp8 unaligned")
    out, lse = gpu_fp8(w, A)
    ref_o, ref_l = oracle_fp8(w)
    compare(out, lse, ref_o, ref_l, ATOL_FP8, what="fp8_unaligned", lse_atol=LSE_ATOL_FP8)


@pytest.mark.parametrize("hq,hkv,d,bs", [(8, 8, 128, 16), (32, 1, 128, 16), (12, 4, 64, 32),
                                         (64, 2, 128, 64)])
def test_decode_group_sizes(A, hq, hkv, d, bs):
    """GQA groups 1, 32 (the largest decode takes), 3 (not a power of two)
    and 32 at block size 64; ragged lengths incl. 0 and a split boundary."""
    w = W.make_decode("decg", 34, "bf16", [1, 0, 257, 4096, 1500], hq, hkv, d, bs)
    banner(f"decode groups hq={hq} hkv={hkv} d={d} bs={bs}")
    out, lse = gpu_decode(w, A, split_tokens=1024)
    ref_o, ref_l = oracle_decode(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"decode_g{hq // hkv}_d{d}_bs{bs}")
