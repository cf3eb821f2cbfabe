"""GPU invariants of the attention path that hold whatever the inputs.

* GQA equals explicit head expansion: query head h reads kv head
  h // (Hq / Hkv) (the onnxruntime PR "[CUDA] PagedAttention: add SM<80 fp16
  fallback via memory-efficient attention", Implementation, step 2: "GQA
  head expansion"), so repeating each K/V head Hq / Hkv times and calling
  with num_kv_heads = Hq must give the GQA call's result.  The kernels keep
  each row's running max per row and the key tiles aligned alike, so the
  two calls agree bit for bit (causal, unmasked and patch masks, where the
  key tiles start at key 0 in both).
* A packed sequence under the document mask equals the same documents as
  separate sequences of one cu_seqlens batch (same PR, Implementation,
  step 3: varlen packing is the document separator), within the parity
  bars (the key tiles fall differently, so the float sums differ in order).
* Canaries: 16-byte-aligned guard regions around out and lse keep their
  bit patterns after prefill, block-sparse prefill, decode and fp8 calls
  (no write outside the rows the call owns).
"""

import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import (ATOL_16, ATOL_FP8, DEV, LSE_ATOL, LSE_ATOL_FP8, REL_16, banner,
                        gpu_cache, gpu_fp8, gpu_prefill, lib_module, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _i32(a):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32).to(DEV)


def _expanded(w):
    """The same workload with every K/V head repeated Hq / Hkv times."""
    g = w.num_heads // w.num_kv_heads
    return dataclasses.replace(w, num_kv_heads=w.num_heads,
                               k_new=w.k_new.repeat_interleave(g, dim=1).contiguous(),
                               v_new=w.v_new.repeat_interleave(g, dim=1).contiguous())


@pytest.mark.parametrize("case", ["causal", "cross_no_mask", "patch", "causal_d64_fp16"])
def test_gqa_equals_head_expansion_bitwise(A, case):
    if case == "causal":
        w = W.make_prefill("gx", 301, "bf16", [300, 77, 513], [300, 77, 513], 16, 4, 128, 16,
                           W.MASK_CAUSAL)
    elif case == "cross_no_mask":
        w = W.make_prefill("gx", 302, "bf16", [130, 5, 260], [300, 700, 33], 32, 8, 128, 32,
                           W.MASK_NONE)
    elif case == "patch":
        w = W.byte_patch_cross_bf16(batch=2, n_bytes=600, n_keys=90, seed=303)
        w = dataclasses.replace(w, num_kv_heads=4,
                                k_new=w.k_new[:, :4].contiguous(), v_new=w.v_new[:, :4].contiguous())
    else:
        w = W.make_prefill("gx", 304, "f16", [200, 129], [200, 129], 8, 1, 64, 16, W.MASK_CAUSAL)
    banner(f"GQA expansion {case}: H={w.num_heads}/{w.num_kv_heads}")
    out_g, lse_g = gpu_prefill(w, A)
    we = _expanded(w)
    out_e, lse_e = gpu_prefill(we, A)
    assert torch.equal(out_g, out_e), "GQA and expanded outputs differ"
    assert torch.equal(lse_g, lse_e), "GQA and expanded LSE differ"


def test_fp8_gqa_equals_head_expansion_bitwise(A):
    w = W.make_fp8("gx8", 305, [300, 77, 513], [300, 77, 513], 16, 4, 128, W.MASK_CAUSAL)
    banner("fp8 GQA expansion")
    out_g, lse_g = gpu_fp8(w, A)
    g = w.num_heads // w.num_kv_heads
    we = dataclasses.replace(w, num_kv_heads=w.num_heads,
                             k_new=w.k_new.repeat_interleave(g, dim=1).contiguous(),
                             v8_colmajor=w.v8_colmajor.repeat_interleave(g, dim=0).contiguous())
    out_e, lse_e = gpu_fp8(we, A)
    assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e)


def _doc_layout(lens):
    ids = np.concatenate([np.full(n, i, np.int32) for i, n in enumerate(lens)])
    return ids


@pytest.mark.parametrize("doc_lens", [[100, 37, 200, 1, 64], [513, 300]])
def test_document_packed_equals_split(A, doc_lens):
    total = int(sum(doc_lens))
    ids = _doc_layout(doc_lens)
    packed = W.make_prefill("dp", 306, "bf16", [total], [total], 8, 2, 128, 16,
                            W.MASK_DOCUMENT | W.MASK_CAUSAL, q_ids=ids, kv_ids=ids)
    split = W.make_prefill("ds", 306, "bf16", doc_lens, doc_lens, 8, 2, 128, 16, W.MASK_CAUSAL)
    split = dataclasses.replace(split, q=packed.q, k_new=packed.k_new, v_new=packed.v_new)
    banner(f"document packed vs split {doc_lens}")
    out_p, lse_p = gpu_prefill(packed, A)
    out_s, lse_s = gpu_prefill(split, A)
    d = (out_p.float() - out_s.float()).abs()
    print(f"[invariant] packed vs split: max-abs {float(d.max()):.3e}, "
          f"lse {float((lse_p - lse_s).abs().max()):.3e}", flush=True)
    assert float(d.max()) <= ATOL_16
    assert float(d.norm() / out_s.float().norm()) <= REL_16
    assert float((lse_p - lse_s).abs().max()) <= LSE_ATOL


def test_fp8_document_packed_equals_split(A):
    doc_lens = [100, 37, 200, 1, 64]
    total = int(sum(doc_lens))
    ids = _doc_layout(doc_lens)
    packed = W.make_fp8("dp8", 307, [total], [total], 8, 2, 128, W.MASK_DOCUMENT | W.MASK_CAUSAL,
                        q_ids=ids, kv_ids=ids)
    split = dataclasses.replace(packed, q_lens=np.asarray(doc_lens, np.int32),
                                kv_lens=np.asarray(doc_lens, np.int32),
                                new_lens=np.zeros(len(doc_lens), np.int32),
                                block_table=np.zeros((len(doc_lens), 1), np.int32),
                                mask_flags=W.MASK_CAUSAL, q_ids=None, kv_ids=None)
    banner("fp8 document packed vs split")
    out_p, lse_p = gpu_fp8(packed, A)
    out_s, lse_s = gpu_fp8(split, A)
    assert float((out_p.float() - out_s.float()).abs().max()) <= ATOL_FP8
    assert float((lse_p - lse_s).abs().max()) <= LSE_ATOL_FP8


# ----------------------------------------------------------------- canaries

PAD = 256   # guard elements on each side (a multiple of 16 bytes for every dtype)


def _guarded(shape, dtype, fill_bits):
    """A tensor of `shape` inside a buffer with PAD guard elements on each
    side, all filled with the bit pattern fill_bits; returns (view, buffer)."""
    n = int(np.prod(shape))
    itype = {2: torch.int16, 4: torch.int32}[torch.empty(0, dtype=dtype).element_size()]
    buf = torch.full((n + 2 * PAD,), fill_bits, dtype=itype, device=DEV).view(dtype)
    return buf[PAD:PAD + n].view(shape), buf


def _guards_intact(buf, fill_bits, what):
    itype = torch.int16 if buf.element_size() == 2 else torch.int32
    raw = buf.view(itype)
    assert bool((raw[:PAD] == fill_bits).all()), f"{what}: bytes before the output changed"
    assert bool((raw[-PAD:] == fill_bits).all()), f"{what}: bytes after the output changed"


def test_canaries_prefill_decode_fp8(A):
    banner("canaries")
    CAN16, CAN32 = 0x5A5A, 0x5A5A5A5A
    # paged prefill (causal, ragged) and its block-sparse variant
    w = W.make_prefill("cn", 308, "bf16", [300, 77, 1, 129], [300, 77, 1, 129], 8, 2, 128, 16,
                       W.MASK_CAUSAL)
    kc, vc, bt, cu_kv = gpu_cache(w, A)
    cu_q = A.attn_cu_seqlens(_i32(w.q_lens))
    out, ob = _guarded(tuple(w.q.shape), torch.bfloat16, CAN16)
    lse, lb = _guarded((w.total_q, w.num_heads), torch.float32, CAN32)
    A.attn_paged_prefill_fwd(w.q.to(DEV), kc, vc, bt, cu_q, cu_kv, int(w.q_lens.max()),
                             int(w.kv_lens.max()), scale=w.scale, mask_flags=w.mask_flags,
                             out=out, lse=lse)
    torch.cuda.synchronize()
    _guards_intact(ob, CAN16, "prefill out")
    _guards_intact(lb, CAN32, "prefill lse")
    ref = A.attn_paged_prefill_fwd(w.q.to(DEV), kc, vc, bt, cu_q, cu_kv, int(w.q_lens.max()),
                                   int(w.kv_lens.max()), scale=w.scale, mask_flags=w.mask_flags)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)

    kn, ki, fn, fi = W.causal_block_mask(w.q_lens, w.kv_lens, 64, 64)
    out, ob = _guarded(tuple(w.q.shape), torch.bfloat16, CAN16)
    lse, lb = _guarded((w.total_q, w.num_heads), torch.float32, CAN32)
    A.attn_paged_prefill_block_sparse_fwd(
        w.q.to(DEV), kc, vc, bt, cu_q, cu_kv, int(w.q_lens.max()), int(w.kv_lens.max()), 64, 64,
        _i32(kn), _i32(ki), _i32(fn), _i32(fi), scale=w.scale, mask_flags=w.mask_flags, out=out,
        lse=lse)
    torch.cuda.synchronize()
    _guards_intact(ob, CAN16, "block-sparse out")
    _guards_intact(lb, CAN32, "block-sparse lse")

    # decode, several splits per sequence
    wd = W.make_decode("cnd", 309, "bf16", [1, 0, 700, 3000], 16, 2, 128, 16)
    kc, vc, bt, cu_kv = gpu_cache(wd, A)
    out, ob = _guarded(tuple(wd.q.shape), torch.bfloat16, CAN16)
    lse, lb = _guarded((wd.batch, wd.num_heads), torch.float32, CAN32)
    A.attn_paged_decode_fwd(wd.q.to(DEV), kc, vc, bt, cu_kv, int(wd.kv_lens.max()),
                            scale=wd.scale, split_tokens=512, out=out, lse=lse)
    torch.cuda.synchronize()
    _guards_intact(ob, CAN16, "decode out")
    _guards_intact(lb, CAN32, "decode lse")

    # dense fp8
    w8 = W.make_fp8("cn8", 310, [300, 77, 13], [300, 77, 130], 8, 2, 128, W.MASK_CAUSAL)
    cq, ck = A.attn_cu_seqlens(_i32(w8.q_lens)), A.attn_cu_seqlens(_i32(w8.kv_lens))
    out, ob = _guarded((w8.total_q, w8.num_heads, 128), torch.bfloat16, CAN16)
    lse, lb = _guarded((w8.total_q, w8.num_heads), torch.float32, CAN32)
    A.attn_fp8_fwd(w8.q.to(DEV), w8.k_new.to(DEV), w8.v8_colmajor.to(DEV),
                   torch.as_tensor(w8.descale, dtype=torch.float32).to(DEV), cq, ck,
                   int(w8.q_lens.max()), int(w8.kv_lens.max()), scale=w8.scale,
                   mask_flags=w8.mask_flags, out=out, lse=lse)
    torch.cuda.synchronize()
    _guards_intact(ob, CAN16, "fp8 out")
    _guards_intact(lb, CAN32, "fp8 lse")
