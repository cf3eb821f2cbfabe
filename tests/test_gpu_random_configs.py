"""Seeded random configurations of the paged prefill and the decode against
the fp64 oracle.

Each case draws its own head counts (GQA group sizes 1-16, kv head counts
that give every decode head grouping), head size, 16-bit type, block size,
ragged lengths with empty sequences, mask, local window, score cap and forced
split size, so that combinations no hand-written case names are held to the
same bars as the others; the dense fp8 prefill draws its heads, layout, mask,
window, cap and the sign of its scale the same way.  The draws are fixed by their seeds: a failure names
its case and reruns identically.
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import (ATOL_16, ATOL_FP8, LSE_ATOL_FP8, REL_16, banner, compare,
                        draw_masked_lengths, gpu_cache, gpu_decode, gpu_decode_fp8kv, gpu_fp8,
                        gpu_prefill, lib_module, oracle_decode, oracle_decode_fp8kv, oracle_fp8,
                        oracle_prefill, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]

N_CASES = 24
MASKS = [W.MASK_NONE, W.MASK_CAUSAL, W.MASK_CAUSAL, W.MASK_DOCUMENT,
         W.MASK_DOCUMENT | W.MASK_CAUSAL, W.MASK_PATCH]


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _draw_decode(i):
    rng = np.random.default_rng(7100 + i)
    hkv = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12, 16]))
    g = int(rng.choice([1, 2, 3, 4, 8] if hkv >= 8 else [1, 2, 3, 4, 8, 16]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    bs = int(rng.choice([16, 32, 64]))
    batch = int(rng.integers(1, 10))
    lens = rng.integers(1, 3000, batch)
    lens[rng.random(batch) < 0.2] = 0
    window = int(rng.choice([0, 0, 1, 100, 1000]))
    softcap = float(rng.choice([0.0, 0.0, 5.0, 30.0]))
    split = int(rng.choice([256, 512, 1280]))
    fp8 = bool(rng.random() < 0.3)
    return dict(seed=7200 + i, hq=hkv * g, hkv=hkv, d=d, dtype=dtype, bs=bs, lens=lens,
                window=window, softcap=softcap, split=split, fp8=fp8)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode(A, i):
    c = _draw_decode(i)
    banner(f"random decode {i}: {c['hq']}/{c['hkv']} heads, D {c['d']} {c['dtype']}, block "
           f"{c['bs']}, lens {c['lens'].tolist()}, window {c['window']}, cap {c['softcap']}, "
           f"split {c['split']}, fp8 cache {c['fp8']}")
    w = W.make_decode(f"rdec{i}", c["seed"], c["dtype"], c["lens"], c["hq"], c["hkv"], c["d"],
                      c["bs"])
    if c["fp8"]:
        w = W.to_fp8_cache(w)
        ref_o, ref_l = oracle_decode_fp8kv(w, window=c["window"], softcap=c["softcap"])
        cache = gpu_cache(w, A, poison=0x7F)
        run = gpu_decode_fp8kv
    else:
        ref_o, ref_l = oracle_decode(w, window=c["window"], softcap=c["softcap"])
        cache = gpu_cache(w, A)
        run = gpu_decode
    for st in (0, c["split"]):
        out, lse = run(w, A, split_tokens=st, cache=cache, window=c["window"],
                       softcap=c["softcap"])
        compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"random_decode_{i}_split{st}")


def _draw_prefill(i):
    rng = np.random.default_rng(7300 + i)
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8] if hkv <= 2 else [1, 2, 4]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    bs = int(rng.choice([16, 32, 64]))
    batch = int(rng.integers(1, 5))
    mask, q_lens, kv_lens, q_ids, kv_ids = draw_masked_lengths(rng, batch, 420, 500, MASKS)
    window = int(rng.choice([0, 0, 0, 1, 50, 300]))
    softcap = float(rng.choice([0.0, 0.0, 0.0, 20.0]))
    return dict(seed=7400 + i, hq=hkv * g, hkv=hkv, d=d, dtype=dtype, bs=bs, q_lens=q_lens,
                kv_lens=kv_lens, mask=mask, q_ids=q_ids, kv_ids=kv_ids, window=window,
                softcap=softcap)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_prefill(A, i):
    c = _draw_prefill(i)
    banner(f"random prefill {i}: {c['hq']}/{c['hkv']} heads, D {c['d']} {c['dtype']}, block "
           f"{c['bs']}, q {c['q_lens'].tolist()} kv {c['kv_lens'].tolist()}, mask {c['mask']}, "
           f"window {c['window']}, cap {c['softcap']}")
    w = W.make_prefill(f"rpre{i}", c["seed"], c["dtype"], c["q_lens"], c["kv_lens"], c["hq"],
                       c["hkv"], c["d"], c["bs"], c["mask"], q_ids=c["q_ids"],
                       kv_ids=c["kv_ids"])
    out, lse = gpu_prefill(w, A, window=c["window"], softcap=c["softcap"])
    ref_o, ref_l = oracle_prefill(w, window=c["window"], softcap=c["softcap"])
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"random_prefill_{i}")


def _draw_fp8(i):
    rng = np.random.default_rng(7500 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 5))
    mask, q_lens, kv_lens, q_ids, kv_ids = draw_masked_lengths(rng, batch, 500, 500, MASKS)
    window = int(rng.choice([0, 0, 0, 1, 70, 260]))
    softcap = float(rng.choice([0.0, 0.0, 0.0, 20.0]))
    # scales of the default magnitude 1/sqrt(D) (the workloads' and the bar's),
    # either sign: a sharper softmax (a causal draw at 0.2 reached 0.083)
    # weighs a few keys whose single e4m3 rounding no longer averages out
    scale = rng.choice([None, None, -0.07, 0.09])
    return dict(seed=7600 + i, hq=hkv * g, hkv=hkv, q_lens=q_lens, kv_lens=kv_lens, mask=mask,
                q_ids=q_ids, kv_ids=kv_ids, window=window, softcap=softcap,
                scale=None if scale is None else float(scale))


@pytest.mark.parametrize("i", range(12))
def test_random_fp8(A, i):
    c = _draw_fp8(i)
    banner(f"random fp8 {i}: {c['hq']}/{c['hkv']} heads, q {c['q_lens'].tolist()} "
           f"kv {c['kv_lens'].tolist()}, mask {c['mask']}, window {c['window']}, "
           f"cap {c['softcap']}, scale {c['scale']}")
    w = W.make_fp8(f"r8_{i}", c["seed"], c["q_lens"], c["kv_lens"], c["hq"], c["hkv"], 128,
                   c["mask"], q_ids=c["q_ids"], kv_ids=c["kv_ids"], scale=c["scale"])
    out, lse = gpu_fp8(w, A, window=c["window"], softcap=c["softcap"])
    ref_o, ref_l = oracle_fp8(w, window=c["window"], softcap=c["softcap"])
    compare(out, lse, ref_o, ref_l, ATOL_FP8, what=f"random_fp8_{i}", lse_atol=LSE_ATOL_FP8)
