"""GPU parity of the varlen attention backward against the fp64 oracle.

The GPU chain is the library's own: the paged prefill produces O and the
LSE, the backward takes them with a seeded dO and the packed K / V.  The
oracle differentiates the forward's definition from Q, K, V and dO alone
(no input from the GPU side).

Bars: the forward's fp16/bf16 bars, max-abs 2e-2 and relative L2 1e-2, with
the max-abs bar scaled by the largest reference gradient where that exceeds
1.  The kernel rounds P and dS to the 16-bit type before the MFMA products
(relative 2^-9 per element, bf16) and reads the forward's rounded O for
delta, so its gradients carry about the forward output's relative error.
"""

import numpy as np
import pytest
import torch

import oracle as ORC
import workloads as W
from gpu_common import (DEV, REL_16, banner, draw_masked_lengths, gpu_prefill, lib_module,
                        requires_gpu, sub_workload)

pytestmark = [pytest.mark.gpu, requires_gpu]

ATOL_GRAD = 2e-2


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _i32(a):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32).to(DEV)


def _cmp(got, ref, what):
    g = got.float().cpu().double().numpy()
    assert not np.any(np.isnan(g)), f"{what}: NaN"
    diff = np.abs(g - ref)
    big = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    max_abs = float(diff.max()) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(g - ref) / den) if den > 0 else float(np.linalg.norm(g))
    print(f"[parity] {what}: max-abs {max_abs:.3g} (bar {ATOL_GRAD * big:.3g}), rel-L2 {rel:.3g}",
          flush=True)
    assert max_abs <= ATOL_GRAD * big, what
    assert rel <= REL_16, what


def _backward(A, w, dout, window=0, softcap=0.0):
    out, lse = gpu_prefill(w, A, window=window, softcap=softcap)
    cu_q = A.attn_cu_seqlens(_i32(w.q_lens))
    cu_kv = A.attn_cu_seqlens(_i32(w.kv_lens))
    q_ids = None if w.q_ids is None else _i32(w.q_ids)
    kv_ids = None if w.kv_ids is None else _i32(w.kv_ids)
    grads = A.attn_varlen_bwd(w.q.to(DEV), w.k_new.to(DEV), w.v_new.to(DEV), out, dout.to(DEV),
                              lse, cu_q, cu_kv, int(w.q_lens.max(initial=0)),
                              int(w.kv_lens.max(initial=0)), scale=w.scale,
                              mask_flags=w.mask_flags, q_ids=q_ids, kv_ids=kv_ids, window=window,
                              softcap=softcap)
    torch.cuda.synchronize()
    return grads


def _oracle(w, dout, window=0, softcap=0.0):
    return ORC.attention_varlen_bwd(w.q.double().cpu().numpy(), w.k_new.double().cpu().numpy(),
                                    w.v_new.double().cpu().numpy(),
                                    dout.double().cpu().numpy(), ORC.cu_seqlens(w.q_lens),
                                    ORC.cu_seqlens(w.kv_lens), w.scale, w.mask_flags, w.q_ids,
                                    w.kv_ids, window, softcap)


def _case(A, w, seed, what, window=0, softcap=0.0):
    banner(f"backward {what}: q={w.q_lens.tolist()} kv={w.kv_lens.tolist()} "
           f"H={w.num_heads}/{w.num_kv_heads} D={w.head_size} mask={w.mask_flags} "
           f"window={window} softcap={softcap} {w.dtype}")
    dout = W.make_dout(seed, w)
    dq, dk, dv = _backward(A, w, dout, window, softcap)
    rq, rk, rv = _oracle(w, dout, window, softcap)
    _cmp(dq, rq, f"{what} dq")
    _cmp(dk, rk, f"{what} dk")
    _cmp(dv, rv, f"{what} dv")


def test_causal_gqa_bf16(A):
    w = W.make_prefill("bw1", 121, "bf16", [300, 200, 129], [300, 200, 129], 8, 2, 128, 16,
                       W.MASK_CAUSAL, device=DEV)
    _case(A, w, 122, "causal_gqa_bf16")


def test_causal_window_d64_fp16(A):
    w = W.make_prefill("bw2", 123, "f16", [65, 190], [65, 190], 16, 2, 64, 32, W.MASK_CAUSAL,
                       device=DEV)
    _case(A, w, 124, "causal_window_d64_fp16", window=50)


def test_cross_q_shorter_no_mask(A):
    w = W.make_prefill("bw3", 125, "bf16", [40, 130], [333, 400], 8, 2, 128, 16, 0, device=DEV)
    _case(A, w, 126, "cross_no_mask")


def test_document_causal_with_empty_rows(A):
    """Document ids where the last query document has no keys: those rows
    get dq = 0 and add nothing to dk, dv."""
    rng = np.random.default_rng(127)
    ql, kl = [300, 180], [300, 170]
    qd, kd = [], []
    for a, b in zip(ql, kl):
        cuts = np.sort(rng.choice(np.arange(1, b), 3, replace=False))
        kd.append(np.searchsorted(cuts, np.arange(b), side="right").astype(np.int32))
        qi = np.searchsorted(cuts, np.arange(a), side="right").astype(np.int32)
        qi[-7:] = 9          # a document with no keys
        qd.append(qi)
    w = W.make_prefill("bw4", 128, "bf16", ql, kl, 8, 4, 128, 16, W.MASK_DOCUMENT,
                       q_ids=np.concatenate(qd), kv_ids=np.concatenate(kd), device=DEV)
    _case(A, w, 129, "document_empty_rows")


def test_patch_cross_d64(A):
    w = W.byte_patch_cross_bf16(device=DEV, batch=2, n_bytes=700, n_keys=96, seed=130)
    _case(A, w, 131, "byte_patch_cross")


@pytest.mark.parametrize("i", range(10))
def test_random_configs(A, i):
    """Seeded random layouts: heads and GQA group, head size, dtype, ragged and
    empty sequences, mask (none, causal, document, document + causal, patch),
    window and cap drawn per case."""
    rng = np.random.default_rng(7700 + i)
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f16"]))
    batch = int(rng.integers(1, 4))
    masks = [W.MASK_NONE, W.MASK_CAUSAL, W.MASK_CAUSAL, W.MASK_DOCUMENT,
             W.MASK_DOCUMENT | W.MASK_CAUSAL, W.MASK_PATCH]
    mask, q_lens, kv_lens, q_ids, kv_ids = draw_masked_lengths(rng, batch, 300, 300, masks)
    window = int(rng.choice([0, 0, 1, 60]))
    softcap = float(rng.choice([0.0, 0.0, 15.0]))
    w = W.make_prefill(f"bwr{i}", 7800 + i, dtype, q_lens, kv_lens, hkv * g, hkv, d, 16, mask,
                       q_ids=q_ids, kv_ids=kv_ids, device=DEV)
    _case(A, w, 7900 + i, f"random_{i}", window=window, softcap=softcap)


def test_full_varlen_causal_sampled(A):
    """The varlen workload: the backward over all 34,805 tokens; the oracle
    re-derives two sequences (the shortest and a seeded one) alone, whose
    dq rows and dk / dv rows must match."""
    w = W.varlen_gqa_causal_bf16(device=DEV)
    banner(f"backward {w.name}: total_q {w.total_q}")
    dout = W.make_dout(132, w)
    dq, dk, dv = _backward(A, w, dout)
    lens = np.asarray(w.q_lens)
    rng = np.random.default_rng(133)
    seqs = sorted({int(np.argmin(lens)), int(rng.integers(len(lens)))})
    sub, q_idx = sub_workload(w, seqs)
    ck = np.concatenate([[0], np.cumsum(w.kv_lens, dtype=np.int64)])
    kv_idx = np.concatenate([np.arange(ck[b], ck[b + 1]) for b in seqs])
    sub_dout = dout[torch.as_tensor(q_idx, device=dout.device)].cpu()
    rq, rk, rv = ORC.attention_varlen_bwd(
        sub.q.double().numpy(), sub.k_new.double().numpy(), sub.v_new.double().numpy(),
        sub_dout.double().numpy(), ORC.cu_seqlens(sub.q_lens), ORC.cu_seqlens(sub.kv_lens),
        sub.scale, sub.mask_flags)
    gi = torch.as_tensor(q_idx, device=DEV)
    ki = torch.as_tensor(kv_idx, device=DEV)
    _cmp(dq[gi], rq, f"{w.name} seqs {seqs} dq")
    _cmp(dk[ki], rk, f"{w.name} seqs {seqs} dk")
    _cmp(dv[ki], rv, f"{w.name} seqs {seqs} dv")


def test_empty_sequences(A):
    """A sequence with queries but no keys (O = 0, LSE = -inf: dq = 0) and
    one with keys but no queries (dk = dv = 0), next to a normal one."""
    w = W.make_prefill("bw5", 134, "bf16", [0, 50, 30], [20, 0, 30], 8, 2, 128, 16, 0,
                       device=DEV)
    _case(A, w, 135, "empty_sequences")


def test_softcap_causal_gqa_bf16(A):
    """A cap that bends most scores (2.0 at scale 0.5): dS carries 1 - tanh^2."""
    w = W.make_prefill("bw6", 138, "bf16", [300, 129], [300, 129], 8, 2, 128, 16, W.MASK_CAUSAL,
                       device=DEV, scale=0.5)
    _case(A, w, 139, "softcap_causal_gqa_bf16", softcap=2.0)


def test_softcap_window_d64_fp16(A):
    """The pages' cap of 50 with a local window, D = 64, fp16."""
    w = W.make_prefill("bw7", 140, "f16", [65, 190], [65, 190], 16, 2, 64, 32, W.MASK_CAUSAL,
                       device=DEV)
    _case(A, w, 141, "softcap_window_d64_fp16", window=50, softcap=50.0)


def test_document_window_softcap_together(A):
    rng = np.random.default_rng(151)
    lens = [260, 180]
    docs = []
    for n in lens:
        cuts = np.sort(rng.choice(np.arange(1, n), 3, replace=False))
        docs.append(np.searchsorted(cuts, np.arange(n), side="right").astype(np.int32))
    ids = np.concatenate(docs)
    w = W.make_prefill("bw8", 152, "bf16", lens, lens, 8, 2, 128, 16,
                       W.MASK_DOCUMENT | W.MASK_CAUSAL, q_ids=ids, kv_ids=ids, device=DEV)
    _case(A, w, 153, "document_window_softcap", window=60, softcap=3.0)


def test_no_query_rows_gives_zero_dk_dv(A):
    """Every sequence has keys and no query rows (total_q = 0): the empty
    query-side tensors come as NULL pointers, and dK, dV (NaN-filled before
    the call) must come back exactly 0."""
    w = W.make_prefill("bw0q", 181, "bf16", [0, 0, 0], [40, 7, 129], 8, 2, 128, 16,
                       W.MASK_CAUSAL, device=DEV)
    banner(f"backward with no query rows: kv={w.kv_lens.tolist()}")
    cu_q = A.attn_cu_seqlens(_i32(w.q_lens))
    cu_kv = A.attn_cu_seqlens(_i32(w.kv_lens))
    empty = torch.empty((0, w.num_heads, w.head_size), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((0, w.num_heads), dtype=torch.float32, device=DEV)
    dk = torch.full_like(w.k_new, float("nan"))
    dv = torch.full_like(w.v_new, float("nan"))
    dq, dk, dv = A.attn_varlen_bwd(empty, w.k_new, w.v_new, empty, empty, lse, cu_q, cu_kv, 0,
                                   int(w.kv_lens.max()), scale=w.scale, mask_flags=w.mask_flags,
                                   dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert dq.numel() == 0
    assert torch.all(dk == 0) and torch.all(dv == 0)
