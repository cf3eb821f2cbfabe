"""GPU parity of decode over an fp8 e4m3 paged cache against the fp64 oracle.

The cache holds e4m3 codes written by attn_reshape_and_cache into pages
poisoned with NaN codes (0x7F), so a read of a slot no sequence owns shows up
as NaN.  The oracle decodes the same codes, applies (dk, dv) and attends in
fp64.  Widening e4m3 to fp16 / bf16 is exact, so the bars are those of the
16-bit decode.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (ATOL_16, REL_16, banner, compare, gpu_cache, gpu_decode_fp8kv,
                        lib_module, oracle_decode_fp8kv, requires_gpu, sub_workload)

pytestmark = [pytest.mark.gpu, requires_gpu]

DEV = "cuda"


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _fp8kv_decode(seed, dtype, lens, hq, hkv, d, bs):
    return W.to_fp8_cache(W.make_decode("dec8", seed, dtype, lens, hq, hkv, d, bs))


def test_decode_fp8kv_small_and_split_invariance(A):
    w = _fp8kv_decode(81, "bf16", [1, 17, 300, 1000, 2500, 0, 4096], 32, 8, 128, 16)
    banner(f"decode fp8kv small, descale {w.kv_descale.tolist()}")
    cache = gpu_cache(w, A, poison=0x7F)
    ref_o, ref_l = oracle_decode_fp8kv(w)
    for st in (0, 256, 512, 1024, 4096):
        out, lse = gpu_decode_fp8kv(w, A, split_tokens=st, cache=cache)
        compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"decode_fp8kv split={st}")


def test_decode_fp8kv_d64_fp16(A):
    w = _fp8kv_decode(82, "f16", [33, 700, 129], 16, 2, 64, 32)
    banner("decode fp8kv d64 fp16")
    out, lse = gpu_decode_fp8kv(w, A)
    ref_o, ref_l = oracle_decode_fp8kv(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="decode_fp8kv_d64_fp16")


def test_decode_fp8kv_descale_and_scale(A):
    """Descales far from 1 and a negative scale: dk must enter the scores and
    dv the output, each once."""
    w = _fp8kv_decode(83, "bf16", [65, 1200, 31], 8, 2, 128, 16)
    dv0 = float(w.kv_descale[1])     # the quantiser's descale: codes * dv0 ~ N(0, 1)
    w.kv_descale = np.asarray([0.03, 7.5], dtype=np.float32)
    w.scale = -0.9
    banner("decode fp8kv descale (0.03, 7.5), scale -0.9")
    out, lse = gpu_decode_fp8kv(w, A, split_tokens=512)
    ref_o, ref_l = oracle_decode_fp8kv(w)
    # the bars hold for unit-variance V: compare in the units V had before
    # its descale was replaced
    unit = dv0 / 7.5
    compare(out.float() * unit, lse, ref_o * unit, ref_l, ATOL_16, REL_16,
            what="decode_fp8kv_descale")


@pytest.mark.parametrize("window,softcap", [(300, 0.0), (0, 4.0), (1000, 50.0), (1, 0.0)])
def test_decode_fp8kv_window_softcap(A, window, softcap):
    w = _fp8kv_decode(84, "bf16", [1, 17, 300, 1000, 2500, 0, 4096], 32, 8, 128, 16)
    banner(f"decode fp8kv window={window} softcap={softcap}")
    cache = gpu_cache(w, A, poison=0x7F)
    ref_o, ref_l = oracle_decode_fp8kv(w, window=window, softcap=softcap)
    for st in (0, 256):
        out, lse = gpu_decode_fp8kv(w, A, split_tokens=st, cache=cache, window=window,
                                    softcap=softcap)
        compare(out, lse, ref_o, ref_l, ATOL_16, REL_16,
                what=f"decode_fp8kv_w{window}_c{softcap}_split{st}")


def test_full_paged_gqa_decode_fp8kv(A):
    """The 64-sequence paged decode workload with an fp8 cache, in the
    benchmark's launch configuration; sampled sequences against the oracle."""
    w = W.paged_gqa_decode_fp8kv(device=DEV)
    banner(f"{w.name}: {w.total_kv} kv tokens, max {int(w.kv_lens.max())}")
    out, lse = gpu_decode_fp8kv(w, A)
    lens = np.asarray(w.kv_lens)
    rng = np.random.default_rng(85)
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens))}
                  | set(rng.choice(len(lens), size=6, replace=False).tolist()))
    sub, q_idx = sub_workload(w, seqs, decode=True)
    ref_o, ref_l = oracle_decode_fp8kv(sub)
    g = torch.as_tensor(q_idx, device=out.device)
    compare(out[g], lse[g], ref_o, ref_l, ATOL_16, REL_16,
            what=f"{w.name} seqs {seqs} x {w.num_heads} heads")


@pytest.mark.parametrize("hq,hkv,d,bs", [(32, 1, 128, 16), (12, 4, 64, 64)])
def test_decode_fp8kv_group_sizes(A, hq, hkv, d, bs):
    w = _fp8kv_decode(86, "bf16", [1, 0, 257, 4096, 1500], hq, hkv, d, bs)
    banner(f"decode fp8kv groups hq={hq} hkv={hkv} d={d} bs={bs}")
    out, lse = gpu_decode_fp8kv(w, A, split_tokens=1024)
    ref_o, ref_l = oracle_decode_fp8kv(w)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what=f"decode_fp8kv_g{hq // hkv}_d{d}")


def test_decode_fp8kv_d64_fp16_window_softcap(A):
    w = _fp8kv_decode(87, "f16", [33, 700, 129, 0], 16, 2, 64, 32)
    w.scale = 0.5
    banner("decode fp8kv d64 fp16 window 100 softcap 2")
    out, lse = gpu_decode_fp8kv(w, A, window=100, softcap=2.0)
    ref_o, ref_l = oracle_decode_fp8kv(w, window=100, softcap=2.0)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="decode_fp8kv_d64_fp16_w100_c2")
