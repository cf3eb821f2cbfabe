"""GPU parity of the fused rotary + packed-QKV unpack + cache write against
the fp64 oracle, and of attention on its output.

The pages name the three steps (the onnxruntime PR, section Implementation,
step 1, and its Testing axes rotary on/off, rotary_interleaved on/off,
packed-QKV on/off); the oracle's module docstring states how they are read.

Bars: the kernel rotates in fp32 and rounds once, the oracle rotates in fp64,
so a rotated element is within one unit in the last place of the 16-bit type
of the oracle's value plus fp32's error on a c - b s, 2^-23 (|a| + |b|)
(``_check_rotated``); unrotated features and V are copied bit for bit;
cache slots no token owns keep their NaN poison.  Attention on the rotated
tensors meets the usual fp16/bf16 bars against the oracle's fp64 chain.
"""

import numpy as np
import pytest
import torch

import oracle as ORC
import workloads as W
from gpu_common import (ATOL_16, DEV, REL_16, banner, compare, lib_module, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]

_TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _i32(a):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32).to(DEV)


def _layout(seed, new_lens, kv_lens, bs):
    rng = np.random.default_rng(seed)
    table, nb = W._block_table(rng, kv_lens, bs)
    return table, nb


def _ulp16(x, dtype):
    """Spacing of the 16-bit type at |x| (normal range; subnormal floor)."""
    mant, emin = (7, -126) if dtype == "bf16" else (10, -14)
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - mant)


def _pair_magnitude(x, rd, interleaved):
    """|a| + |b| of the rotation pair each feature belongs to (|x| past rd)."""
    m = np.abs(np.asarray(x, dtype=np.float64))
    out = m.copy()
    if rd:
        j = np.arange(rd)
        partner = (j ^ 1) if interleaved else (j + rd // 2) % rd
        out[..., :rd] = m[..., :rd] + m[..., partner]
    return out


def _check_rotated(got, ref, x, rd, interleaved, dtype, what):
    """|got - ref| <= ulp16(ref) + 2^-23 (|a| + |b|): one rounding to the
    16-bit type (half an ulp, a whole one when it crosses a binade) plus
    fp32's error on a c - b s (each product and the sum rounded once, |c|,
    |s| <= 1), which matters where the pair nearly cancels."""
    g = got.float().cpu().double().numpy()
    err = np.abs(g - ref)
    bound = _ulp16(ref, dtype) + 2.0 ** -23 * _pair_magnitude(x, rd, interleaved)
    ratio = err / bound
    k = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else None
    if k is not None:
        print(f"[parity] {what}: max error {float(ratio[k]):.3f} of the bound "
              f"(ref {ref[k]:.6g}, got {g[k]:.6g}, |a|+|b| "
              f"{_pair_magnitude(x, rd, interleaved)[k]:.4g})", flush=True)
    assert np.all(err <= bound), f"{what}: error above the bound"


def _run(A, seed, dtype, new_lens, kv_lens, hq, hkv, d, bs, rd, interleaved, packed,
         in_place=False):
    """Fill a NaN-poisoned cache through the fused kernel and through the
    oracle; compare q_out and every cache slot.  Returns what the attention
    cases need."""
    new_lens = np.asarray(new_lens, np.int32)
    kv_lens = np.asarray(kv_lens, np.int32)
    total = int(new_lens.sum())
    table, nb = _layout(seed, new_lens, kv_lens, bs)
    qkv = W.make_packed_qkv(seed, dtype, total, hq, hkv, d, device=DEV)
    cos, sin = W.rope_tables(int(kv_lens.max()) + 3, max(rd, 16))
    banner(f"rotary {dtype} new={new_lens.tolist()} kv={kv_lens.tolist()} H={hq}/{hkv} D={d} "
           f"rd={rd} interleaved={interleaved} packed={packed} in_place={in_place}")
    shape = (nb, bs, hkv, d)
    kc = torch.full(shape, float("nan"), dtype=_TDT[dtype], device=DEV)
    vc = torch.full(shape, float("nan"), dtype=_TDT[dtype], device=DEV)
    bt = _i32(table)
    cu_new = A.attn_cu_seqlens(_i32(new_lens))
    cu_kv = A.attn_cu_seqlens(_i32(kv_lens))
    ct = torch.from_numpy(cos).to(DEV) if rd else None
    st = torch.from_numpy(sin).to(DEV) if rd else None
    q3, k3, v3 = (t.contiguous() for t in torch.split(
        qkv.view(total, hq + 2 * hkv, d), [hq, hkv, hkv], dim=1))
    if packed:
        q_out = A.attn_rotary_reshape_and_cache(kc, vc, bt, cu_new, cu_kv, int(kv_lens.max()),
                                                qkv=qkv, num_heads=hq, cos_table=ct, sin_table=st,
                                                rotary_dim=rd, interleaved=interleaved)
    else:
        q_in = q3.clone()
        q_out = A.attn_rotary_reshape_and_cache(kc, vc, bt, cu_new, cu_kv, int(kv_lens.max()),
                                                q=q_in, k=k3, v=v3, cos_table=ct, sin_table=st,
                                                rotary_dim=rd, interleaved=interleaved,
                                                q_out=q_in if in_place else None)
    torch.cuda.synchronize()
    # oracle
    x = qkv.double().cpu().numpy()
    oq, ok, ov = ORC.unpack_qkv(x, hq, hkv, d)
    ocu_new, ocu_kv = ORC.cu_seqlens(new_lens), ORC.cu_seqlens(kv_lens)
    okc = np.full(shape, np.nan)
    ovc = np.full(shape, np.nan)
    rq, okc, ovc = ORC.rotary_reshape_and_cache(oq, ok, ov, cos, sin, rd, interleaved, okc, ovc,
                                                table, ocu_new, ocu_kv, bs)
    _check_rotated(q_out, rq, oq, rd, interleaved, dtype, "q_out")
    kg = kc.float().cpu().double().numpy()
    vg = vc.float().cpu().double().numpy()
    owned = ~np.isnan(okc[..., 0, 0])
    assert np.array_equal(np.isnan(kg[..., 0, 0]), ~owned), "K written outside the owned slots"
    assert np.array_equal(np.isnan(vg[..., 0, 0]), ~owned), "V written outside the owned slots"
    k_src = np.full(shape, np.nan)
    _, k_src, _ = ORC.rotary_reshape_and_cache(oq, ok, ov, cos, sin, 0, False, k_src,
                                               np.full(shape, np.nan), table, ocu_new, ocu_kv, bs)
    _check_rotated(kc[torch.from_numpy(owned).to(DEV)], okc[owned], k_src[owned], rd, interleaved,
                   dtype, "k_cache")
    # V and the features past rotary_dim are copies
    assert np.array_equal(vg[owned], ovc[owned]), "V not copied bit for bit"
    if rd < d:
        assert np.array_equal(q_out[..., rd:].float().cpu().double().numpy(), oq[..., rd:])
        assert np.array_equal(kg[owned][..., rd:], okc[owned][..., rd:])
    return dict(q=q_out, kc=kc, vc=vc, bt=bt, cu_kv=cu_kv, new_lens=new_lens, kv_lens=kv_lens,
                table=table, bs=bs, rq=rq, okc=okc, ovc=ovc)


@pytest.mark.parametrize("interleaved", [False, True])
def test_packed_full_rotary_bf16(A, interleaved):
    # a prefill, a decode step, a chunk appended to a longer sequence
    _run(A, 111, "bf16", [37, 1, 20], [37, 50, 300], 8, 2, 128, 16, 128, interleaved, True)


@pytest.mark.parametrize("interleaved", [False, True])
def test_separate_partial_rotary_f16_in_place(A, interleaved):
    _run(A, 112, "f16", [64, 3, 129], [64, 90, 129], 16, 4, 64, 32, 32, interleaved, False,
         in_place=True)


def test_no_rotary_is_unpack_and_cache(A):
    r = _run(A, 113, "bf16", [100, 17], [100, 40], 4, 4, 128, 64, 0, False, True)
    assert r is not None


def _round16(x, dtype):
    """The oracle's values as the 16-bit cache / q_out holds them (RNE)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(_TDT[dtype]).double().numpy()


def test_rotary_then_prefill_and_decode(A):
    """Rotated Q and cache into the causal paged prefill, and a decode step
    whose single token sits at kv_len - 1, against the oracle's chain.  The
    cache and q_out hold 16-bit values, so the chain's attention runs on the
    oracle's rotated values rounded to that type."""
    r = _run(A, 114, "bf16", [300, 200, 129], [300, 200, 129], 8, 2, 128, 16, 128, False, True)
    cu_q = A.attn_cu_seqlens(_i32(r["new_lens"]))
    out, lse = A.attn_paged_prefill_fwd(r["q"], r["kc"], r["vc"], r["bt"], cu_q, r["cu_kv"], 300,
                                        300, scale=1.0 / np.sqrt(128), mask_flags=W.MASK_CAUSAL,
                                        return_lse=True)
    torch.cuda.synchronize()
    ocu = ORC.cu_seqlens(r["kv_lens"])
    ref_o, ref_l = ORC.paged_attention(_round16(r["rq"], "bf16"), _round16(r["okc"], "bf16"),
                                       r["ovc"], r["table"], ocu, ocu, r["bs"],
                                       1.0 / np.sqrt(128), ORC.MASK_CAUSAL)
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="rotary -> prefill")

    # decode: the whole cache comes through the fused kernel; each sequence's
    # query is its last rotated row (position kv_len - 1)
    d = _run(A, 115, "bf16", [700, 33, 1], [700, 33, 1], 32, 8, 128, 16, 64, True, True)
    last = np.cumsum(d["kv_lens"]) - 1
    q_dec = d["q"][torch.as_tensor(last, device=DEV)].contiguous()
    out, lse = A.attn_paged_decode_fwd(q_dec, d["kc"], d["vc"], d["bt"], d["cu_kv"], 700,
                                       return_lse=True)
    torch.cuda.synchronize()
    ocu = ORC.cu_seqlens(d["kv_lens"])
    ref_o, ref_l = ORC.paged_decode(_round16(d["rq"][last], "bf16"), _round16(d["okc"], "bf16"),
                                    d["ovc"], d["table"], ocu, d["bs"], 1.0 / np.sqrt(128))
    compare(out, lse, ref_o, ref_l, ATOL_16, REL_16, what="rotary -> decode")
