"""GPU parity at the full workload sizes the benchmark times, in the same
launch configuration (default tile shapes, automatic decode split), on
sampled outputs that the fp64 oracle computes one by one.

Sampling: a few whole sequences (the longest, the shortest and seeded random
ones) are re-derived on the oracle side from the same generated tokens; within
them, each sequence's first rows (one visible key under causal masking), its
middle and last row and seeded random rows are compared for every head.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (ATOL_16, ATOL_FP8, LSE_ATOL_FP8, REL_16, banner, compare, gpu_decode,
                        gpu_fp8, gpu_prefill, lib_module, oracle_decode, oracle_fp8,
                        oracle_prefill, requires_gpu, sample_rows, sub_fp8, sub_workload)

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _pick_seqs(lens, n_random, seed):
    lens = np.asarray(lens)
    pick = {int(np.argmax(lens)), int(np.argmin(lens))}
    rng = np.random.default_rng(seed)
    pick |= set(rng.choice(len(lens), size=min(n_random, len(lens)), replace=False).tolist())
    return sorted(pick)


def test_full_varlen_gqa_causal_bf16(A):
    w = W.varlen_gqa_causal_bf16(device=DEV)
    banner(f"{w.name}: total_q {w.total_q}, max len {int(w.q_lens.max())}")
    out, lse = gpu_prefill(w, A)
    seqs = _pick_seqs(w.q_lens, 2, 71)
    sub, q_idx = sub_workload(w, seqs)
    rows = sample_rows(sub.q_lens, 40, 72)
    ref_o, ref_l = oracle_prefill(sub, rows)
    g = torch.as_tensor(q_idx[rows], device=out.device)
    compare(out[g], lse[g], ref_o[rows], ref_l[rows], ATOL_16, REL_16,
            what=f"{w.name} seqs {seqs}, {len(rows)} rows x {w.num_heads} heads")


def test_full_paged_gqa_decode_bf16(A):
    w = W.paged_gqa_decode_bf16(device=DEV)
    banner(f"{w.name}: {w.total_kv} kv tokens, max {int(w.kv_lens.max())}")
    out, lse = gpu_decode(w, A)
    seqs = _pick_seqs(w.kv_lens, 6, 73)
    sub, q_idx = sub_workload(w, seqs, decode=True)
    ref_o, ref_l = oracle_decode(sub)
    g = torch.as_tensor(q_idx, device=out.device)
    compare(out[g], lse[g], ref_o, ref_l, ATOL_16, REL_16,
            what=f"{w.name} seqs {seqs} x {w.num_heads} heads")


def test_full_byte_patch_cross_bf16(A):
    w = W.byte_patch_cross_bf16(device=DEV)
    banner(f"{w.name}: patches {w.extra['patch_counts']}")
    out, lse = gpu_prefill(w, A)
    rows = sample_rows(w.q_lens, 96, 74)
    ref_o, ref_l = oracle_prefill(w, rows)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, rows=rows,
            what=f"{w.name}, {len(rows)} rows x {w.num_heads} heads")


def test_full_dense_causal_fp8(A):
    w = W.dense_causal_fp8(device=DEV)
    banner(f"{w.name}")
    out, lse = gpu_fp8(w, A)
    for b in range(w.batch):
        sub, q_idx = sub_fp8(w, [b])
        # the first 32 rows (1 to 32 visible keys), then sampled ones
        rows = np.union1d(np.arange(32), sample_rows(sub.q_lens, 24, 75 + b))
        ref_o, ref_l = oracle_fp8(sub, rows)
        g = torch.as_tensor(q_idx[rows], device=out.device)
        compare(out[g], lse[g], ref_o[rows], ref_l[rows], ATOL_FP8, what=f"{w.name} seq {b}",
                lse_atol=LSE_ATOL_FP8)


# ------------------------------------------------------------ edge cases

@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 16, 8, 2), (64, 32, 4, 4)])
def test_prefill_keys_beyond_one_page_window(A, d, bs, hq, hkv):
    """kv_len 20000: more pages than the kernel stages at once (512 block ids),
    so the key range is walked in several windows; bottom-right causal."""
    w = W.make_prefill("longkv", 41, "bf16", [200, 37], [20000, 9000], hq, hkv, d, bs,
                       W.MASK_CAUSAL)
    banner(f"long kv d{d} bs{bs}")
    out, lse = gpu_prefill(w, A)
    ref_o, ref_l = oracle_prefill(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"long_kv_d{d}_bs{bs}")


def test_prefill_zero_length_sequences(A):
    """Sequences with no queries, or no keys, inside a batch."""
    w = W.make_prefill("zeros", 42, "bf16", [100, 0, 50, 30], [100, 40, 50, 0], 8, 2, 128, 16,
                       W.MASK_CAUSAL)
    out, lse = gpu_prefill(w, A)
    ref_o, ref_l = oracle_prefill(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="zero_length_sequences")


def test_prefill_many_sequences(A):
    """300 short ragged sequences x 8 head groups: 2400 (sequence, head group)
    units, so each XCD walks its units in several chunks of 64 when it maps
    workgroups to tiles (the varlen workload has 16 units per XCD)."""
    rng = np.random.default_rng(143)
    lens = rng.integers(0, 200, 300)
    w = W.make_prefill("many", 144, "bf16", lens, lens, 32, 8, 128, 16, W.MASK_CAUSAL, rng=rng)
    banner(f"many sequences: {len(lens)}, total {int(lens.sum())}")
    out, lse = gpu_prefill(w, A)
    ref_o, ref_l = oracle_prefill(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="many_sequences")


def test_fp8_many_sequences(A):
    """200 short causal sequences (many units per XCD): every row, from the
    one-key first rows on, within the fp8 bar."""
    rng = np.random.default_rng(145)
    lens = rng.integers(0, 300, 200)
    w = W.make_fp8("many8", 146, lens, lens, 8, 2, 128, W.MASK_CAUSAL)
    banner(f"fp8 many sequences: {len(lens)}, total {int(lens.sum())}")
    out, lse = gpu_fp8(w, A)
    ref_o, ref_l = oracle_fp8(w)
    compare(out, lse, ref_o, ref_l, ATOL_FP8, what="fp8_many_sequences", lse_atol=LSE_ATOL_FP8)


def test_decode_many_sequences(A):
    rng = np.random.default_rng(147)
    lens = rng.integers(0, 600, 600)
    w = W.make_decode("manyd", 148, "bf16", lens, 32, 8, 128, 16)
    banner(f"decode many sequences: {len(lens)}")
    out, lse = gpu_decode(w, A)
    ref_o, ref_l = oracle_decode(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="decode_many_sequences")
