"""HIP-graph capture of the hot path through the C ABI.

Three call sequences are captured once each with torch.cuda.graph and then
replayed with new inputs copied in (eagerly) between replays:
  * a whole prefill step: cu_seqlens of q and kv, the paged cache write, the
    paged causal prefill with LSE;
  * a split-KV decode (decode and combine kernels) with the caller's
    workspace;
  * a varlen backward (the dQ kernel with its row sums, then dK/dV) with the caller's
    workspace and gradient buffers.
Every replay must equal an eager call on the same inputs bit for bit: the
kernels, launch shapes and reduction orders are the same, and the library
allocates nothing and records no memset, so the graphs hold kernel nodes
only.  Consecutive replays must also differ (the replay really ran on the
new inputs), and nothing may be NaN (torch.equal fails on NaN).
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import DEV, banner, lib_module, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

_REPLAYS = 3


@pytest.fixture(scope="module")
def A():
    return lib_module()


def _i32(a):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32).to(DEV)


def _capture(fn):
    """Warm fn up on a side stream (library and allocator set-up), then
    capture one call; returns the graph and the captured call's outputs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    return g, outs


def _fresh(gen, t):
    """New values for input t (same shape and dtype), drawn on the device."""
    return torch.randn(t.shape, generator=gen, device=DEV, dtype=torch.float32).to(t.dtype)


def _replays_match_eager(g, g_outs, fn, refresh, what):
    prev = None
    for r in range(_REPLAYS):
        refresh()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in g_outs]
        ref = fn()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"{what}: replay {r} output {i} differs from the eager call"
        if prev is not None:
            assert not torch.equal(prev, got[0]), f"{what}: replay {r} repeated the previous output"
        prev = got[0]
        print(f"[graph] {what}: replay {r} equals the eager call", flush=True)


def test_prefill_step_graph(A):
    w = W.make_prefill("graph_prefill", 171, "bf16", [300, 1, 517, 64], [300, 1, 517, 64], 8, 2,
                       128, 16, W.MASK_CAUSAL, device=DEV)
    banner(f"graph prefill step: q={w.q_lens.tolist()} H={w.num_heads}/{w.num_kv_heads} D=128")
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    bt = _i32(w.block_table)
    lens_q, lens_kv = _i32(w.q_lens), _i32(w.kv_lens)
    cu_q = torch.empty(len(w.q_lens) + 1, dtype=torch.int32, device=DEV)
    cu_kv = torch.empty_like(cu_q)
    q, k_new, v_new = w.q.clone(), w.k_new.clone(), w.v_new.clone()
    mq, mk = int(w.q_lens.max()), int(w.kv_lens.max())

    def step():
        A.attn_cu_seqlens(lens_q, out=cu_q)
        A.attn_cu_seqlens(lens_kv, out=cu_kv)
        A.attn_reshape_and_cache(k_new, v_new, kc, vc, bt, cu_kv, cu_kv)
        return A.attn_paged_prefill_fwd(q, kc, vc, bt, cu_q, cu_kv, mq, mk, scale=w.scale,
                                        mask_flags=w.mask_flags, return_lse=True)

    g, outs = _capture(step)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(172)

    def refresh():
        q.copy_(_fresh(gen, q))
        k_new.copy_(_fresh(gen, k_new))
        v_new.copy_(_fresh(gen, v_new))
        kc.fill_(float("nan"))   # the replay must write the cache again
        vc.fill_(float("nan"))

    _replays_match_eager(g, outs, step, refresh, "prefill step")


def test_decode_graph(A):
    w = W.make_decode("graph_decode", 173, "bf16", [700, 33, 4096, 1], 32, 8, 128, 16, device=DEV)
    banner(f"graph decode: kv={w.kv_lens.tolist()} H=32/8 D=128")
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    bt = _i32(w.block_table)
    cu_kv = A.attn_cu_seqlens(_i32(w.kv_lens))
    A.attn_reshape_and_cache(w.k_new, w.v_new, kc, vc, bt, cu_kv, cu_kv)
    mk = int(w.kv_lens.max())
    q = w.q.clone()
    ws = torch.empty(A.attn_paged_decode_workspace_bytes(w.batch, w.num_heads, w.num_kv_heads,
                                                         w.head_size, mk),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)

    def call():
        o, lse = A.attn_paged_decode_fwd(q, kc, vc, bt, cu_kv, mk, scale=w.scale, out=out,
                                         workspace=ws, return_lse=True)
        return o.clone(), lse

    g, outs = _capture(call)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(174)
    _replays_match_eager(g, outs, call, lambda: q.copy_(_fresh(gen, q)), "decode")


def test_backward_graph(A):
    w = W.make_prefill("graph_bwd", 175, "bf16", [260, 1, 390], [260, 1, 390], 8, 2, 128, 16,
                       W.MASK_CAUSAL, device=DEV)
    banner(f"graph backward: q={w.q_lens.tolist()} H={w.num_heads}/{w.num_kv_heads} D=128")
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    bt = _i32(w.block_table)
    cu = A.attn_cu_seqlens(_i32(w.q_lens))
    mq = int(w.q_lens.max())
    q, k, v = w.q.clone(), w.k_new.clone(), w.v_new.clone()
    dout = W.make_dout(176, w).to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty((w.total_q, w.num_heads), dtype=torch.float32, device=DEV)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(max(A.attn_varlen_bwd_workspace_bytes(w.total_q, w.num_heads), 256),
                     dtype=torch.uint8, device=DEV)

    def forward():
        A.attn_reshape_and_cache(k, v, kc, vc, bt, cu, cu)
        o, l = A.attn_paged_prefill_fwd(q, kc, vc, bt, cu, cu, mq, mq, scale=w.scale,
                                        mask_flags=w.mask_flags, return_lse=True)
        out.copy_(o)
        lse.copy_(l)

    def call():
        dq, dk, dv = A.attn_varlen_bwd(q, k, v, out, dout, lse, cu, cu, mq, mq, scale=w.scale,
                                       mask_flags=w.mask_flags, dq=grads[0], dk=grads[1],
                                       dv=grads[2], workspace=ws)
        return dq.clone(), dk.clone(), dv.clone()

    forward()
    g, outs = _capture(call)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(177)

    def refresh():
        q.copy_(_fresh(gen, q))
        k.copy_(_fresh(gen, k))
        v.copy_(_fresh(gen, v))
        dout.copy_(_fresh(gen, dout))
        forward()   # eager: O and LSE of the new inputs

    _replays_match_eager(g, outs, call, refresh, "backward")
