"""torch-facing wrappers of the C ABI: argument marshalling only.

Each function checks that the tensors are contiguous device tensors of the
expected dtype, reads sizes from their shapes, allocates outputs with torch
when the caller gives none, and calls the C entry point of the same name on
torch's current stream.  Every step of the computation runs in the HIP
kernels; nothing here computes on the CPU.
"""

import ctypes
import math

import torch

from . import _lib

_DT = {torch.float16: _lib.ATTN_F16, torch.bfloat16: _lib.ATTN_BF16}


def library_path():
    return _lib.LIB_PATH


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _lse_out(lse, return_lse, shape, dev):
    """The LSE output: the caller's float32 tensor of the given shape, or a new
    one when return_lse is set, or None."""
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=dev) if return_lse else None
    _need(lse, "lse", torch.float32, dev)
    if tuple(lse.shape) != tuple(shape):
        raise ValueError(f"lse must be {list(shape)}")
    return lse


def _u8(t):
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def attn_cu_seqlens(seqlens, out=None):
    """int32 [batch] lengths -> int32 [batch + 1] cumulative lengths (device)."""
    _need(seqlens, "seqlens", torch.int32)
    batch = seqlens.numel()
    if out is None:
        # the kernel writes every entry; an empty batch launches nothing, so
        # its single 0 comes from the allocation
        alloc = torch.zeros if batch == 0 else torch.empty
        out = alloc(batch + 1, dtype=torch.int32, device=seqlens.device)
    _need(out, "out", torch.int32, seqlens.device)
    if out.numel() != batch + 1:
        raise ValueError("out must hold batch + 1 elements")
    lib = _lib.load()
    with torch.cuda.device(seqlens.device):
        _lib.check("attn_cu_seqlens",
                   lib.attn_cu_seqlens(_ptr(seqlens), _ptr(out), batch, _stream(seqlens.device)))
    return out


def attn_reshape_and_cache(k, v, k_cache, v_cache, block_table, cu_seqlens_new, cu_seqlens_kv):
    """Write k, v [total_new, Hkv, D] into the paged caches [NB, bs, Hkv, D] in place."""
    dev = k.device
    for name, t in (("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, device=dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_new", cu_seqlens_new),
                    ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    if not (k.dtype == v.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("k, v and the caches must share a dtype")
    dtype = _DT.get(k.dtype, _lib.ATTN_FP8_E4M3 if k.element_size() == 1 else None)
    if dtype is None:
        raise TypeError(f"unsupported dtype {k.dtype}")
    total_new, hkv, d = k.shape
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    if tuple(k_cache.shape[2:]) != (hkv, d) or v_cache.shape != k_cache.shape or v.shape != k.shape:
        raise ValueError("cache / token shapes disagree")
    batch = cu_seqlens_new.numel() - 1
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_reshape_and_cache", lib.attn_reshape_and_cache(
            _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            block_table.shape[1], _ptr(cu_seqlens_new), _ptr(cu_seqlens_kv), batch, total_new,
            hkv, d, bs, nb, dtype, _stream(dev)))


def attn_varlen_bwd_workspace_bytes(total_q, num_heads):
    return int(_lib.load().attn_varlen_bwd_workspace_bytes(int(total_q), int(num_heads)))


def attn_varlen_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
                    max_seqlen_kv, scale=None, mask_flags=0, q_ids=None, kv_ids=None, window=0,
                    softcap=0.0, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of varlen attention: q, out, dout [total_q, Hq, D],
    k, v [total_kv, Hkv, D] (packed, 16-bit), lse float32 [total_q, Hq] from
    the forward."""
    dev = q.device
    _need(q, "q", (torch.float16, torch.bfloat16))
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need(t, name, q.dtype, dev)
    _need(lse, "lse", torch.float32, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    for name, t in (("q_ids", q_ids), ("kv_ids", kv_ids)):
        if t is not None:
            _need(t, name, torch.int32, dev)
    total_q, hq, d = q.shape
    total_kv, hkv, _ = k.shape
    if v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape or k.shape[2] != d:
        raise ValueError("q / k / v / out / dout shapes disagree")
    if tuple(lse.shape) != (total_q, hq):
        raise ValueError("lse must be [total_q, num_heads]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _need(t, name, q.dtype, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{name} shape")
    lib = _lib.load()
    need = attn_varlen_bwd_workspace_bytes(total_q, hq)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    batch = cu_seqlens_q.numel() - 1
    with torch.cuda.device(dev):
        _lib.check("attn_varlen_bwd", lib.attn_varlen_bwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(cu_seqlens_q),
            _ptr(cu_seqlens_kv), batch, total_q, total_kv, int(max_seqlen_q), int(max_seqlen_kv),
            hq, hkv, d, float(scale), int(mask_flags), _ptr(q_ids), _ptr(kv_ids), int(window),
            float(softcap), _DT[q.dtype], _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            workspace.numel(),
            _stream(dev)))
    return dq, dk, dv


def attn_rotary_reshape_and_cache(k_cache, v_cache, block_table, cu_seqlens_new, cu_seqlens_kv,
                                  max_seqlen_kv, qkv=None, num_heads=None, q=None, k=None, v=None,
                                  cos_table=None, sin_table=None, rotary_dim=None,
                                  interleaved=False, q_out=None, write_q=True):
    """Rotary + packed-QKV unpack + cache write of the new tokens.

    Either qkv [total_new, (num_heads + 2 Hkv) * D] (num_heads required) or
    k, v [total_new, Hkv, D] and optionally q [total_new, Hq, D].  cos_table /
    sin_table float32 [max_position, rotary_dim / 2]; rotary_dim defaults to
    their full width (0 without tables).  Returns the rotated q
    [total_new, Hq, D] (q_out, allocated when not given), or None when no
    query is written."""
    dev = k_cache.device
    nb, bs, hkv, d = k_cache.shape
    _need(k_cache, "k_cache", (torch.float16, torch.bfloat16))
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes differ")
    for name, t in (("block_table", block_table), ("cu_seqlens_new", cu_seqlens_new),
                    ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    if qkv is not None:
        _need(qkv, "qkv", k_cache.dtype, dev)
        if num_heads is None:
            raise ValueError("num_heads is required with packed qkv")
        total = qkv.shape[0]
        if qkv.dim() != 2 or qkv.shape[1] != (num_heads + 2 * hkv) * d:
            raise ValueError("qkv must be [total_new, (num_heads + 2 * num_kv_heads) * head_size]")
        hq = num_heads
    else:
        for name, t in (("k", k), ("v", v)):
            _need(t, name, k_cache.dtype, dev)
        total = k.shape[0]
        if tuple(k.shape) != (total, hkv, d) or v.shape != k.shape:
            raise ValueError("k / v shapes disagree with the cache")
        if q is not None:
            _need(q, "q", k_cache.dtype, dev)
            if q.shape[0] != total or q.shape[2] != d:
                raise ValueError("q shape disagrees")
            hq = q.shape[1]
        else:
            hq = num_heads if num_heads is not None else hkv
    has_q = qkv is not None or q is not None
    if write_q and has_q and q_out is None:
        q_out = torch.empty((total, hq, d), dtype=k_cache.dtype, device=dev)
    if not (write_q and has_q):
        q_out = None
    if q_out is not None:
        _need(q_out, "q_out", k_cache.dtype, dev)
    if rotary_dim is None:
        rotary_dim = 0 if cos_table is None else 2 * cos_table.shape[1]
    max_pos = 0
    if cos_table is not None:
        for name, t in (("cos_table", cos_table), ("sin_table", sin_table)):
            _need(t, name, torch.float32, dev)
        if sin_table.shape != cos_table.shape:
            raise ValueError("cos / sin tables differ in shape")
        max_pos = cos_table.shape[0]
    batch = cu_seqlens_new.numel() - 1
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_rotary_reshape_and_cache", lib.attn_rotary_reshape_and_cache(
            _ptr(qkv), _ptr(q), _ptr(k), _ptr(v), _ptr(cos_table), _ptr(sin_table), max_pos,
            int(rotary_dim), int(bool(interleaved)), _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), block_table.shape[1], _ptr(cu_seqlens_new), _ptr(cu_seqlens_kv),
            batch, total, int(max_seqlen_kv), hq, hkv, d, bs, nb, _DT[k_cache.dtype],
            _stream(dev)))
    return q_out


def attn_paged_prefill_fwd(q, k_cache, v_cache, block_table, cu_seqlens_q, cu_seqlens_kv,
                           max_seqlen_q, max_seqlen_kv, scale=None, mask_flags=0, q_ids=None,
                           kv_ids=None, out=None, return_lse=False, window=0, softcap=0.0, lse=None):
    """Paged varlen attention; returns out (and lse [total_q, Hq] fp32 if asked).
    window: local window in keys (0 = none); softcap: score cap (0 = none)."""
    dev = q.device
    _need(q, "q", (torch.float16, torch.bfloat16))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, q.dtype, dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    for name, t in (("q_ids", q_ids), ("kv_ids", kv_ids)):
        if t is not None:
            _need(t, name, torch.int32, dev)
    total_q, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    if dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes disagree with q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    lse = _lse_out(lse, return_lse, (total_q, hq), dev)
    batch = cu_seqlens_q.numel() - 1
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_paged_prefill_fwd", lib.attn_paged_prefill_fwd(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
            _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), batch, total_q, int(max_seqlen_q),
            int(max_seqlen_kv), hq, hkv, d, bs, nb, float(scale), int(mask_flags), _ptr(q_ids),
            _ptr(kv_ids), int(window), float(softcap), _DT[q.dtype], _ptr(out), _ptr(lse),
            _stream(dev)))
    return (out, lse) if lse is not None else out


def attn_paged_prefill_block_sparse_fwd(q, k_cache, v_cache, block_table, cu_seqlens_q,
                                        cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, q_block,
                                        kv_block, kv_num_blocks, kv_indices,
                                        full_kv_num_blocks=None, full_kv_indices=None,
                                        scale=None, mask_flags=0, q_ids=None, kv_ids=None,
                                        out=None, return_lse=False, window=0, softcap=0.0, lse=None):
    """Paged varlen attention under a stored block-sparse mask: kv_num_blocks
    int32 [batch, Hm, n_qb], kv_indices int32 [batch, Hm, n_qb, capacity]
    (Hm = 1, num_kv_heads or num_heads); the full pair is optional."""
    dev = q.device
    _need(q, "q", (torch.float16, torch.bfloat16))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, q.dtype, dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_kv", cu_seqlens_kv), ("kv_num_blocks", kv_num_blocks),
                    ("kv_indices", kv_indices)):
        _need(t, name, torch.int32, dev)
    for name, t in (("q_ids", q_ids), ("kv_ids", kv_ids), ("full_kv_num_blocks", full_kv_num_blocks),
                    ("full_kv_indices", full_kv_indices)):
        if t is not None:
            _need(t, name, torch.int32, dev)
    if (full_kv_num_blocks is None) != (full_kv_indices is None):
        raise ValueError("full_kv_num_blocks and full_kv_indices go together")
    batch = cu_seqlens_q.numel() - 1
    if kv_num_blocks.dim() != 3 or kv_num_blocks.shape[0] != batch:
        raise ValueError("kv_num_blocks must be [batch, mask_heads, num_q_blocks]")
    hm, n_qb = kv_num_blocks.shape[1], kv_num_blocks.shape[2]
    if kv_indices.dim() != 4 or tuple(kv_indices.shape[:3]) != (batch, hm, n_qb):
        raise ValueError("kv_indices must be [batch, mask_heads, num_q_blocks, capacity]")
    cap = kv_indices.shape[3]
    if full_kv_num_blocks is not None and (tuple(full_kv_num_blocks.shape) != (batch, hm, n_qb)
                                           or tuple(full_kv_indices.shape) != tuple(kv_indices.shape)):
        raise ValueError("the full lists must have the partial lists' shapes")
    total_q, hq, d = q.shape
    nb, bs, hkv, dk = k_cache.shape
    if dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes disagree with q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    lse = _lse_out(lse, return_lse, (total_q, hq), dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_paged_prefill_block_sparse_fwd", lib.attn_paged_prefill_block_sparse_fwd(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
            _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), batch, total_q, int(max_seqlen_q),
            int(max_seqlen_kv), hq, hkv, d, bs, nb, float(scale), int(mask_flags), _ptr(q_ids),
            _ptr(kv_ids), int(window), float(softcap), int(q_block), int(kv_block), hm, n_qb, cap,
            _ptr(kv_num_blocks), _ptr(kv_indices), _ptr(full_kv_num_blocks),
            _ptr(full_kv_indices), _DT[q.dtype], _ptr(out), _ptr(lse), _stream(dev)))
    return (out, lse) if lse is not None else out


def attn_paged_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_size, max_seqlen_kv,
                                      split_tokens=0, window=0):
    return int(_lib.load().attn_paged_decode_workspace_bytes(
        batch, num_heads, num_kv_heads, head_size, int(max_seqlen_kv), int(window),
        int(split_tokens)))


def attn_paged_decode_fwd(q, k_cache, v_cache, block_table, cu_seqlens_kv, max_seqlen_kv,
                          scale=None, split_tokens=0, out=None, return_lse=False, workspace=None,
                          window=0, softcap=0.0, lse=None):
    """One query per sequence (q [batch, Hq, D]) against the paged cache.
    window: keep each sequence's last `window` keys (0 = all); softcap: score cap."""
    dev = q.device
    _need(q, "q", (torch.float16, torch.bfloat16))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, q.dtype, dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    batch, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_paged_decode_workspace_bytes(batch, hq, hkv, d, max_seqlen_kv, split_tokens, window)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    lse = _lse_out(lse, return_lse, (batch, hq), dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_paged_decode_fwd", lib.attn_paged_decode_fwd(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
            _ptr(cu_seqlens_kv), batch, int(max_seqlen_kv), hq, hkv, d, bs, nb, float(scale),
            int(window), float(softcap), int(split_tokens), _DT[q.dtype], _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream(dev)))
    return (out, lse) if lse is not None else out


def attn_paged_decode_fwd_noalloc(q, k_cache, v_cache, block_table, cu_seqlens_kv, max_seqlen_kv,
                                  scale=None, split_tokens=0, out=None, return_lse=False,
                                  window=0, softcap=0.0, lse=None):
    """attn_paged_decode_fwd without a workspace: the split partials live in
    the library's per-GPU scratch array, so the C call allocates nothing
    (pass `out` / `lse` to keep this wrapper from allocating them).  Calls
    that overlap in time on one GPU race on that scratch."""
    dev = q.device
    _need(q, "q", (torch.float16, torch.bfloat16))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, q.dtype, dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    batch, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    lse = _lse_out(lse, return_lse, (batch, hq), dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_paged_decode_fwd_noalloc", lib.attn_paged_decode_fwd_noalloc(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
            _ptr(cu_seqlens_kv), batch, int(max_seqlen_kv), hq, hkv, d, bs, nb, float(scale),
            int(window), float(softcap), int(split_tokens), _DT[q.dtype], _ptr(out), _ptr(lse),
            _stream(dev)))
    return (out, lse) if lse is not None else out


def attn_paged_decode_fp8kv_fwd(q, k_cache8, v_cache8, kv_descale, block_table, cu_seqlens_kv,
                                max_seqlen_kv, scale=None, split_tokens=0, out=None,
                                return_lse=False, workspace=None, window=0, softcap=0.0, lse=None):
    """Decode against an fp8 e4m3 paged cache: k_cache8 / v_cache8 uint8 (or
    float8_e4m3fn) [num_blocks, block_size, Hkv, D], kv_descale fp32 [2]
    (dk, dv); q [batch, Hq, D] fp16 or bf16."""
    dev = q.device
    _need(q, "q", (torch.float16, torch.bfloat16))
    k8, v8 = _u8(k_cache8), _u8(v_cache8)
    for name, t in (("k_cache8", k8), ("v_cache8", v8)):
        _need(t, name, torch.uint8, dev)
    if v8.shape != k8.shape:
        raise ValueError("k_cache8 and v_cache8 shapes differ")
    _need(kv_descale, "kv_descale", torch.float32, dev)
    if kv_descale.numel() != 2:
        raise ValueError("kv_descale must hold (dk, dv)")
    for name, t in (("block_table", block_table), ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    batch, hq, d = q.shape
    nb, bs, hkv, _ = k8.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_paged_decode_workspace_bytes(batch, hq, hkv, d, max_seqlen_kv, split_tokens, window)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    lse = _lse_out(lse, return_lse, (batch, hq), dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_paged_decode_fp8kv_fwd", lib.attn_paged_decode_fp8kv_fwd(
            _ptr(q), _ptr(k8), _ptr(v8), _ptr(kv_descale), _ptr(block_table), block_table.shape[1],
            _ptr(cu_seqlens_kv), batch, int(max_seqlen_kv), hq, hkv, d, bs, nb, float(scale),
            int(window), float(softcap), int(split_tokens), _DT[q.dtype], _ptr(out), _ptr(lse),
            _ptr(workspace), workspace.numel(), _stream(dev)))
    return (out, lse) if lse is not None else out


def attn_fp8_fwd(q8, k8, v8_colmajor, descale, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
                 max_seqlen_kv, scale=None, mask_flags=0, q_ids=None, kv_ids=None, out=None,
                 return_lse=False, window=0, softcap=0.0, lse=None):
    """fp8 e4m3 attention: q8 [total_q, Hq, D], k8 [total_kv, Hkv, D],
    v8_colmajor [Hkv, D, total_kv] (uint8 codes or float8_e4m3fn), descale fp32 [3]."""
    dev = q8.device
    q8, k8, v8 = _u8(q8), _u8(k8), _u8(v8_colmajor)
    for name, t in (("q8", q8), ("k8", k8), ("v8_colmajor", v8)):
        _need(t, name, torch.uint8, dev)
    _need(descale, "descale", torch.float32, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        _need(t, name, torch.int32, dev)
    for name, t in (("q_ids", q_ids), ("kv_ids", kv_ids)):
        if t is not None:
            _need(t, name, torch.int32, dev)
    total_q, hq, d = q8.shape
    total_kv, hkv, _ = k8.shape
    if tuple(v8.shape) != (hkv, d, total_kv):
        raise ValueError("v8_colmajor must be [Hkv, D, total_kv]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    lse = _lse_out(lse, return_lse, (total_q, hq), dev)
    batch = cu_seqlens_q.numel() - 1
    lib = _lib.load()
    with torch.cuda.device(dev):
        _lib.check("attn_fp8_fwd", lib.attn_fp8_fwd(
            _ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv),
            batch, total_q, total_kv, int(max_seqlen_q), int(max_seqlen_kv), hq, hkv, d,
            float(scale), int(mask_flags), _ptr(q_ids), _ptr(kv_ids), int(window),
            float(softcap), _ptr(out), _ptr(lse), _stream(dev)))
    return (out, lse) if lse is not None else out
