"""fp64 CPU oracle: the plain definition of what the HIP path computes.

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may import it.
Shares no code with the HIP path.  Page tags ([BLT], [ORT], [FLEX], [NANO],
[VLLM]) are defined in ``oracle/__init__.py``.

Everything here is float64 numpy with explicit per-sequence / per-head loops.
A library primitive (a matrix product, ``np.exp``, ``np.max``) serves as a
step; there is no tiling, no online softmax and no reordering beyond the
definition, so each function can be compared with the pages by eye.

Readings where the pages are silent (each is also listed in the design doc):
  * causal alignment when q_len != kv_len is bottom-right: query i of a
    sequence sits at absolute position kv_len - q_len + i, so it sees key j
    iff j <= i + kv_len - q_len.  The pages only show ``q_idx >= kv_idx`` at
    equal lengths ([FLEX] test diff; [NANO] "Note on impact": is_causal at
    Tq == Tk), where both alignments agree.
  * GQA maps q head h to kv head h // (Hq // Hkv) ([FLEX] flex_attention
    docstring: Hq query heads over Hkv key/value heads; [ORT] Implementation,
    step 2: "GQA head expansion").
  * paged cache layout is [num_blocks, block_size, num_kv_heads, head_size]
    ([ORT] Scratch allocation: the size formula multiplies blocks x block_size
    x num_heads x head_size) and block_table is int32 [batch, max_blocks].
  * a query row with no visible key outputs O = 0 and LSE = -inf ([BLT]
    kernel options: ROWS_GUARANTEED_SAFE is False, so such rows may occur; the
    value they take is not printed).
  * LSE is the natural-log logsumexp of the scaled, masked scores ([BLT]
    kernel options: OUTPUT_LOGSUMEXP True, PRESCALE_QK False).
  * fp8 is OCP e4m3fn ([FLEX] _enforce_mem_layouts names torch.float8_e4m3fn);
    a tensor's real value is descale * decoded code.
  * local window and softcap: [ORT] Testing lists "local window on/off" and
    "softcap 0/50" as axes of its parity matrix without defining them.  Read
    here as (a) a left window of W keys ending at the query's own position:
    query i sees key j only if j > i + (kv_len - q_len) - W (same bottom-right
    alignment as CAUSAL; W = 0 means no window), and (b) a score cap c > 0
    applied to the scaled score before masking and softmax,
    s -> c * tanh(s / c) (c = 0 means no cap); LSE is taken over the capped
    scores.
  * stored block-sparse masks: [BLT] (FlexAttention lowering arguments) and
    [FLEX] (test graph inputs) show a BlockMask as kv_num_blocks /
    kv_indices, full_kv_num_blocks / full_kv_indices, a Q and a KV block size
    and a mask_mod.  Read for packed varlen sequences as: query block qb of a
    sequence is its rows [qb*QB, (qb+1)*QB), key block kb its keys
    [kb*KB, (kb+1)*KB); for each (sequence, mask head, qb) the first
    kv_num entries of kv_indices are partial blocks, where the element mask
    (the analytic masks above: causal, document, patch, window) decides, and
    the first full_num entries of full_kv_indices are full blocks, visible
    as a whole (the element mask is not evaluated, as FlexAttention skips
    mask_mod there); every other block is invisible.  A block listed in both
    lists counts as full.  Entries outside [0, ceil(kv_len / KB)) and counts
    beyond the list capacity are ignored / clamped.  The mask's head count
    is 1 (shared by all heads), Hkv (one list per kv head) or Hq.
  * rotary and packed QKV: [ORT] Implementation step 1 runs "rotary" and a
    "packed-QKV unpack" before ReshapeAndCache, and [ORT] Testing has
    "rotary on/off", "rotary_interleaved on/off" and "packed-QKV on/off" as
    parity axes; none is defined there.  Read with their usual meanings:
    a packed token row holds the Hq query heads, then the Hkv key heads, then
    the Hkv value heads; rotary rotates the first rotary_dim features of
    every Q and K head by angle tables indexed by the token's position in its
    sequence (the new token i of a sequence sits at kv_len - n_new + i, where
    reshape_and_cache puts it): non-interleaved pairs feature j with
    j + rotary_dim/2, interleaved pairs 2j with 2j+1; each pair (a, b) goes
    to (a cos - b sin, b cos + a sin) with the table entry j; features past
    rotary_dim and V are unchanged.
  * backward: [BLT] sets OUTPUT_LOGSUMEXP (the forward saves LSE) and the
    [VLLM] review shows the varlen function's backward returning dq, dk, dv;
    the gradients themselves are not printed.  They are those of the
    forward's definition above: with P the masked softmax, O = P V and an
    upstream dO, dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dP * P)),
    dQ = scale dS K, dK = scale dS^T Q; GQA sums dK and dV over the query
    heads of a kv head; a row with no visible key contributes nothing.  With
    a score cap c the score is c tanh(scale q.k / c), so dS is multiplied by
    its derivative 1 - tanh^2 before the dQ and dK products.
"""

import collections

import math

import numpy as np

MASK_CAUSAL = 1
MASK_DOCUMENT = 2
MASK_PATCH = 4

# Which pin covers which function (test names in tests/test_oracle_pins.py).
PIN_STATUS = {
    "cu_seqlens": "pinned: numpy.cumsum special case, hand-written golden example",
    "reshape_and_cache": "pinned: hand-written golden placement example, gather round trip",
    "gather_paged": "pinned: identity table equals packed layout; permuted tables agree",
    "visibility": "pinned: np.tril closed forms, page predicate q_idx >= kv_idx, brute-force counts, "
                  "window bands from np.tril/np.triu",
    "attention_varlen": "pinned: torch CPU fp64 SDPA (dense, GQA, banded window mask), closed forms "
                        "(incl. saturated softcap), invariants",
    "paged_attention": "pinned: equals attention_varlen on gathered K/V; block-table permutation invariance",
    "block_visibility": "pinned: np.kron block expansion, every block partial equals the element mask, "
                        "causal block lists give np.tril, full blocks override the element mask",
    "attention_varlen(block_mask)": "pinned: torch CPU fp64 SDPA with the np.kron-built mask, per-head "
                                    "lists (Hm = 1, Hkv, Hq) against per-head SDPA",
    "paged_decode": "pinned: equals the last row of a causal prefill over the same cache; a window "
                    "equals decode over the cache cut to its last W keys",
    "paged_decode_fp8kv": "pinned: equals paged_decode on caches decoded by torch.float8_e4m3fn; "
                          "hand-derived two-key example with distinct dk, dv; constant-V closed form",
    "unpack_qkv": "pinned: numpy.split of the packed row, hand-written golden row",
    "new_token_positions": "pinned: hand-written golden positions (prefill, decode, chunked prefill)",
    "rotary": "pinned: hand-derived 90-degree example for both pairings, complex multiplication "
              "(interleaved) and the half-split permutation (non-interleaved), norm preservation, "
              "relative-position invariance of q.k",
    "rotary_reshape_and_cache": "pinned: composition of the pinned steps; decode position = kv_len - 1",
    "attention_varlen_bwd": "pinned: torch.autograd through CPU fp64 SDPA with explicit masks (GQA, causal, "
                            "window, document, q shorter than kv) and through composed capped attention, "
                            "central finite differences (with and without a cap), fully masked rows give "
                            "zero gradients",
    "e4m3_decode": "pinned: all 256 codes against torch.float8_e4m3fn; closed-form extremes",
    "fp8_attention": "pinned: equals attention_varlen on decoded values; hand-derived two-key example",
    "default_scale": "pinned: golden value 0.0625 at E=256 from [BLT]",
}


def default_scale(head_size):
    """Softmax scale when the caller gives none: 1/sqrt(E).

    [FLEX] flex_attention docstring, argument ``scale``; the [BLT] lowering
    arguments show the instance 0.0625 for E = 256.
    """
    return 1.0 / math.sqrt(head_size)


def cu_seqlens(seqlens):
    """Cumulative sequence lengths: cu[0] = 0, cu[b + 1] = cu[b] + seqlens[b].

    [ORT] Implementation, steps 1 and 3: the cumulative-seqlens buffer is the
    varlen ``seqstart`` array and its last element is the token total.
    Returns int32 [batch + 1]; raises if the total does not fit int32.
    """
    out = [0]
    for n in seqlens:
        n = int(n)
        if n < 0:
            raise ValueError("negative sequence length")
        out.append(out[-1] + n)
    if out[-1] >= 2**31:
        raise OverflowError("total length does not fit int32")
    return np.asarray(out, dtype=np.int32)


def unpack_qkv(qkv, num_heads, num_kv_heads, head_size):
    """Split packed rows [tokens, (Hq + 2 Hkv) * D] into q [tokens, Hq, D],
    k and v [tokens, Hkv, D] (module docstring: rotary and packed QKV)."""
    x = np.asarray(qkv)
    x = x.reshape(x.shape[0], num_heads + 2 * num_kv_heads, head_size)
    return (x[:, :num_heads], x[:, num_heads:num_heads + num_kv_heads],
            x[:, num_heads + num_kv_heads:])


def new_token_positions(cu_new, cu_kv):
    """Position in its sequence of every new token: kv_len - n_new + i, the
    slot reshape_and_cache writes it to ([ORT] Implementation, step 1)."""
    pos = []
    for b in range(len(cu_new) - 1):
        n_new = int(cu_new[b + 1]) - int(cu_new[b])
        kv_len = int(cu_kv[b + 1]) - int(cu_kv[b])
        pos.extend(range(kv_len - n_new, kv_len))
    return np.asarray(pos, dtype=np.int64)


def rotary(x, positions, cos_table, sin_table, rotary_dim, interleaved):
    """Rotary embedding of x [tokens, H, D] (module docstring), fp64.

    cos_table, sin_table: [max_position, rotary_dim / 2]; token t uses row
    positions[t].  Features at or past rotary_dim are copied.
    """
    out = np.array(x, dtype=np.float64, copy=True)
    if rotary_dim == 0:
        return out
    half = rotary_dim // 2
    c = np.asarray(cos_table, dtype=np.float64)[positions][:, None, :half]
    s = np.asarray(sin_table, dtype=np.float64)[positions][:, None, :half]
    xd = np.asarray(x, dtype=np.float64)
    if interleaved:
        a, b = xd[..., 0:rotary_dim:2], xd[..., 1:rotary_dim:2]
        out[..., 0:rotary_dim:2] = a * c - b * s
        out[..., 1:rotary_dim:2] = b * c + a * s
    else:
        a, b = xd[..., :half], xd[..., half:rotary_dim]
        out[..., :half] = a * c - b * s
        out[..., half:rotary_dim] = b * c + a * s
    return out


def rotary_reshape_and_cache(q, k, v, cos_table, sin_table, rotary_dim, interleaved, k_cache,
                             v_cache, block_table, cu_new, cu_kv, block_size):
    """The preprocessing of [ORT] Implementation step 1 in order: rotary on
    the new tokens' Q and K at their positions, then reshape_and_cache of K
    and V.  Returns (q_rotated, k_cache, v_cache) in fp64."""
    pos = new_token_positions(cu_new, cu_kv)
    qr = rotary(q, pos, cos_table, sin_table, rotary_dim, interleaved)
    kr = rotary(k, pos, cos_table, sin_table, rotary_dim, interleaved)
    kc, vc = reshape_and_cache(kr, np.asarray(v, dtype=np.float64), k_cache, v_cache, block_table,
                               cu_new, cu_kv, block_size)
    return qr, kc, vc


def reshape_and_cache(k_new, v_new, k_cache, v_cache, block_table, cu_new, cu_kv, block_size):
    """Write new K/V tokens into the paged cache (returns updated copies).

    [ORT] Implementation, step 1 (ReshapeAndCache runs before attention) and
    step 2 (block_table maps a sequence's logical blocks to physical blocks).
    Sequence b appends ``n_new = cu_new[b+1] - cu_new[b]`` tokens; after the
    write it holds ``kv_len = cu_kv[b+1] - cu_kv[b]`` tokens, so new token i
    lands at position ``pos = kv_len - n_new + i``, i.e. in physical block
    ``block_table[b][pos // block_size]`` at slot ``pos % block_size``.

    Works on any dtype (the tests pass raw integer views so the copy is
    checked bit for bit).  k_new, v_new: [total_new, Hkv, D];
    caches: [num_blocks, block_size, Hkv, D].
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    batch = len(cu_new) - 1
    for b in range(batch):
        n_new = int(cu_new[b + 1]) - int(cu_new[b])
        kv_len = int(cu_kv[b + 1]) - int(cu_kv[b])
        if n_new > kv_len:
            raise ValueError("sequence has more new tokens than total tokens")
        for i in range(n_new):
            pos = kv_len - n_new + i
            blk = int(block_table[b][pos // block_size])
            slot = pos % block_size
            k_out[blk, slot] = k_new[int(cu_new[b]) + i]
            v_out[blk, slot] = v_new[int(cu_new[b]) + i]
    return k_out, v_out


def gather_paged(cache, table_row, kv_len, block_size):
    """Logical token j of one sequence is ``cache[table_row[j // bs], j % bs]``.

    [ORT] Implementation, step 2: GatherAndExpandPagedKVCache walks block_table
    to build the packed [total_kv_tokens, num_heads, head_size] K/V.
    Returns [kv_len, Hkv, D] (GQA expansion happens in attention_varlen).
    """
    out = np.empty((kv_len,) + tuple(cache.shape[2:]), dtype=cache.dtype)
    for j in range(kv_len):
        out[j] = cache[int(table_row[j // block_size]), j % block_size]
    return out


def visibility(q_len, kv_len, flags, q_ids=None, kv_ids=None, window=0):
    """Boolean [q_len, kv_len]: may query i of a sequence attend to key j.

    Conjunction of
      * CAUSAL:   j <= i + (kv_len - q_len)   ([FLEX] test diff: mask_mod
                  ``q_idx >= kv_idx``; bottom-right when lengths differ)
      * DOCUMENT: q_ids[i] == kv_ids[j]      (document ids; packing several
                  documents into one sequence)
      * PATCH:    j <= q_ids[i]              ([BLT] CrossAttention: byte
                  queries see their own and earlier patch keys; q_ids holds
                  each byte's patch index within its sequence)
      * window W > 0: j > i + (kv_len - q_len) - W  (local window, see the
                  module docstring)
    Every key index j < kv_len exists; there is no other bound.
    """
    if flags & MASK_DOCUMENT and flags & MASK_PATCH:
        raise ValueError("DOCUMENT and PATCH masks are exclusive")
    i = np.arange(q_len)[:, None]
    j = np.arange(kv_len)[None, :]
    vis = np.ones((q_len, kv_len), dtype=bool)
    if flags & MASK_CAUSAL:
        vis &= j <= i + (kv_len - q_len)
    if flags & MASK_DOCUMENT:
        vis &= np.asarray(q_ids)[:q_len, None] == np.asarray(kv_ids)[None, :kv_len]
    if flags & MASK_PATCH:
        vis &= j <= np.asarray(q_ids)[:q_len, None]
    if window > 0:
        vis &= j > i + (kv_len - q_len) - window
    return vis


BlockMask = collections.namedtuple(
    "BlockMask", "q_block kv_block kv_num kv_idx full_num full_idx")
BlockMask.__doc__ = """Stored block-sparse mask (module docstring, last reading).

q_block, kv_block: block sizes in tokens; kv_num: int [batch, Hm, n_qb];
kv_idx: int [batch, Hm, n_qb, cap]; full_num / full_idx the same shapes (or
None: no full blocks)."""


def block_visibility(elem_vis, q_block, kv_block, kv_num, kv_idx, full_num=None, full_idx=None):
    """Boolean [q_len, kv_len] visibility of one sequence under one mask head.

    elem_vis: the element mask ([q_len, kv_len], from ``visibility``), used
    inside partial blocks.  kv_num [n_qb], kv_idx [n_qb, cap] (and the full
    pair) are this sequence's and head's lists.  A full block is visible
    wherever the key exists; a partial block where elem_vis says so.
    """
    q_len, kv_len = elem_vis.shape
    n_kb = -(-kv_len // kv_block)
    out = np.zeros((q_len, kv_len), dtype=bool)
    for qb in range(-(-q_len // q_block)):
        r0, r1 = qb * q_block, min(q_len, (qb + 1) * q_block)
        if qb >= len(kv_num):
            break
        cap = kv_idx.shape[-1]
        for kb in kv_idx[qb][:max(0, min(int(kv_num[qb]), cap))]:
            kb = int(kb)
            if 0 <= kb < n_kb:
                c0, c1 = kb * kv_block, min(kv_len, (kb + 1) * kv_block)
                out[r0:r1, c0:c1] |= elem_vis[r0:r1, c0:c1]
        if full_num is None:
            continue
        for kb in full_idx[qb][:max(0, min(int(full_num[qb]), cap))]:
            kb = int(kb)
            if 0 <= kb < n_kb:
                c0, c1 = kb * kv_block, min(kv_len, (kb + 1) * kv_block)
                out[r0:r1, c0:c1] = True
    return out


def _mask_head(h, hq, hkv, hm):
    """Which of the mask's Hm heads query head h uses (1, Hkv or Hq)."""
    if hm == 1:
        return 0
    if hm == hq:
        return h
    if hm == hkv:
        return h // (hq // hkv)
    raise ValueError("block mask head count must be 1, num_kv_heads or num_heads")


def _softmax_rows(s, vis, v):
    """O = softmax(s restricted to vis) @ v and LSE, row by row (fp64).

    A row with no visible key gives O = 0 and LSE = -inf (reading of [BLT]
    ROWS_GUARANTEED_SAFE False).
    """
    q_len = s.shape[0]
    out = np.zeros((q_len, v.shape[1]), dtype=np.float64)
    lse = np.full(q_len, -np.inf, dtype=np.float64)
    for i in range(q_len):
        idx = np.nonzero(vis[i])[0]
        if idx.size == 0:
            continue
        row = s[i, idx]
        m = row.max()
        w = np.exp(row - m)
        total = w.sum()
        out[i] = (w @ v[idx]) / total
        lse[i] = m + math.log(total)
    return out, lse


def attention_varlen(q, k, v, cu_q, cu_kv, scale, flags=0, q_ids=None, kv_ids=None, rows=None,
                     window=0, softcap=0.0, block_mask=None):
    """Varlen attention over packed (non-paged) K/V, fp64.

    q: [total_q, Hq, D]; k: [total_kv, Hkv, D]; v: [total_kv, Hkv, Dv];
    cu_q, cu_kv: [batch + 1] cumulative lengths ([ORT] Implementation, step 3:
    seqstart_q / seqstart_k, no padding, BSNH strides).
    s[i, j] = scale * <q_i, k_j> with the scale applied to the product
    ([BLT] kernel options: PRESCALE_QK False), masked by ``visibility``, then
    softmax over visible j and the weighted sum of V ([FLEX] flex_attention:
    softmax(scale * QK^T + mask) V).
    q_ids / kv_ids are indexed by global token ([total_q] / [total_kv]).
    rows: optional global query indices to compute (others stay 0 / -inf);
    used to sample outputs of full-size workloads.
    window, softcap: local window and score cap (module docstring); the cap
    acts on the scaled scores before the mask.
    block_mask: optional BlockMask; the element mask then applies inside its
    partial blocks only (``block_visibility``).
    Returns (out [total_q, Hq, Dv], lse [total_q, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    total_q, hq, _ = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    out = np.zeros((total_q, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((total_q, hq), -np.inf, dtype=np.float64)
    want = None if rows is None else np.zeros(total_q, dtype=bool)
    if want is not None:
        want[np.asarray(rows)] = True
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
        q_len, kv_len = q1 - q0, k1 - k0
        sel = np.arange(q_len) if want is None else np.nonzero(want[q0:q1])[0]
        if sel.size == 0:
            continue
        qi = None if q_ids is None else np.asarray(q_ids)[q0:q1]
        ki = None if kv_ids is None else np.asarray(kv_ids)[k0:k1]
        elem = visibility(q_len, kv_len, flags, qi, ki, window)
        vis = elem[sel]
        for h in range(hq):
            kvh = h // group
            if block_mask is not None:
                bm = block_mask
                mh = _mask_head(h, hq, hkv, np.shape(bm.kv_num)[1])
                vis = block_visibility(
                    elem, bm.q_block, bm.kv_block, np.asarray(bm.kv_num)[b, mh],
                    np.asarray(bm.kv_idx)[b, mh],
                    None if bm.full_num is None else np.asarray(bm.full_num)[b, mh],
                    None if bm.full_idx is None else np.asarray(bm.full_idx)[b, mh])[sel]
            s = scale * (q[q0 + sel, h, :] @ k[k0:k1, kvh, :].T)
            if softcap > 0:
                s = softcap * np.tanh(s / softcap)
            o, l = _softmax_rows(s, vis, v[k0:k1, kvh, :])
            out[q0 + sel, h] = o
            lse[q0 + sel, h] = l
    return out, lse


def attention_varlen_bwd(q, k, v, dout, cu_q, cu_kv, scale, flags=0, q_ids=None, kv_ids=None,
                         window=0, softcap=0.0):
    """Gradients of attention_varlen with respect to q, k, v for the upstream
    gradient dout [total_q, Hq, Dv], fp64 (module docstring: backward).  Per
    sequence and head the forward is recomputed from its definition (no LSE
    input), then dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dP * P)),
    times 1 - tanh^2 of the capped score when softcap > 0,
    dQ = scale dS K, dK = scale dS^T Q.
    Returns (dq [total_q, Hq, D], dk [total_kv, Hkv, D], dv [total_kv, Hkv, Dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
        qi = None if q_ids is None else np.asarray(q_ids)[q0:q1]
        ki = None if kv_ids is None else np.asarray(kv_ids)[k0:k1]
        vis = visibility(q1 - q0, k1 - k0, flags, qi, ki, window)
        for h in range(hq):
            kvh = h // group
            Q, K, V, dO = q[q0:q1, h], k[k0:k1, kvh], v[k0:k1, kvh], dout[q0:q1, h]
            raw = scale * (Q @ K.T)
            if softcap > 0:
                th = np.tanh(raw / softcap)
                raw = softcap * th
            s = np.where(vis, raw, -np.inf)
            m = s.max(axis=1, initial=-np.inf, keepdims=True)
            e = np.where(vis, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
            tot = e.sum(axis=1, keepdims=True)
            P = np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)
            dv[k0:k1, kvh] += P.T @ dO
            dP = dO @ V.T
            dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
            if softcap > 0:
                dS = dS * (1.0 - th * th)
            dq[q0:q1, h] = scale * (dS @ K)
            dk[k0:k1, kvh] += scale * (dS.T @ Q)
    return dq, dk, dv


def paged_attention(q, k_cache, v_cache, block_table, cu_q, cu_kv, block_size, scale,
                    flags=0, q_ids=None, kv_ids=None, rows=None, window=0, softcap=0.0,
                    block_mask=None):
    """Attention whose K/V live in a paged cache ([ORT] Implementation, step 2
    then step 3): gather each sequence's K/V through block_table into a packed
    buffer, then run ``attention_varlen`` on it.  Returns (out, lse) in fp64.
    """
    batch = len(cu_kv) - 1
    ks, vs = [], []
    for b in range(batch):
        kv_len = int(cu_kv[b + 1]) - int(cu_kv[b])
        ks.append(gather_paged(k_cache, block_table[b], kv_len, block_size))
        vs.append(gather_paged(v_cache, block_table[b], kv_len, block_size))
    k = np.concatenate(ks, axis=0) if ks else np.zeros((0,) + tuple(k_cache.shape[2:]))
    v = np.concatenate(vs, axis=0) if vs else np.zeros((0,) + tuple(v_cache.shape[2:]))
    return attention_varlen(q, k, v, cu_q, cu_kv, scale, flags, q_ids, kv_ids, rows, window, softcap,
                            block_mask)


def paged_decode(q, k_cache, v_cache, block_table, cu_kv, block_size, scale, batches=None,
                 window=0, softcap=0.0):
    """One new query per sequence (q: [batch, Hq, D]) against its paged cache.

    This is paged_attention with q_len = 1; under bottom-right causal
    alignment the single query sits at the last position and sees every key,
    so no causal mask bites; a window W leaves its last W keys.  ``batches``
    optionally restricts the sequences computed.
    Returns (out [batch, Hq, Dv], lse [batch, Hq]).
    """
    batch = len(cu_kv) - 1
    cu_q = np.arange(batch + 1, dtype=np.int64)
    rows = None if batches is None else np.asarray(batches)
    return paged_attention(q, k_cache, v_cache, block_table, cu_q, cu_kv, block_size, scale,
                           MASK_CAUSAL, rows=rows, window=window, softcap=softcap)


def e4m3_decode(codes):
    """Decode OCP FP8 E4M3 ("fn": finite, no infinities) bytes to float64.

    [FLEX] _enforce_mem_layouts lists torch.float8_e4m3fn among the fp8 dtypes.
    Bit layout s eeee mmm, exponent bias 7.  e = 0 is subnormal:
    m / 8 * 2**-6.  Otherwise (1 + m / 8) * 2**(e - 7), except e = 15, m = 7
    which is NaN.  Largest finite magnitude: 1.75 * 2**8 = 448.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    flat_c = codes.reshape(-1)
    flat_o = out.reshape(-1)
    table = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            table[c] = np.nan
        elif e == 0:
            table[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            table[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    flat_o[:] = table[flat_c]
    return out


def paged_decode_fp8kv(q, k_cache8, v_cache8, kv_descale, block_table, cu_kv, block_size,
                       scale, batches=None, window=0, softcap=0.0):
    """Decode against a paged cache whose K and V hold fp8 e4m3 codes.

    Combines two page features: the paged cache of [ORT] Implementation
    (steps 1-2: tokens placed by reshape_and_cache, found through
    block_table) and the e4m3 storage with per-tensor descales of [FLEX]
    (the real tensor is descale times the decoded code).  The pages do not
    combine them; the plain reading is that the cache holds codes, K is
    dk * code and V is dv * code, and the query (fp16 / bf16) is unchanged.
    k_cache8 / v_cache8: uint8 codes [num_blocks, block_size, Hkv, D];
    kv_descale = (dk, dv).  Everything else as paged_decode.
    """
    dk, dv = (float(x) for x in kv_descale)
    k = dk * e4m3_decode(k_cache8)
    v = dv * e4m3_decode(v_cache8)
    return paged_decode(q, k, v, block_table, cu_kv, block_size, scale, batches, window, softcap)


def fp8_attention(q8, k8, v8_colmajor, descale, cu_q, cu_kv, scale, flags=0,
                  q_ids=None, kv_ids=None, rows=None, window=0, softcap=0.0):
    """fp8 e4m3 attention: decode, apply per-tensor descales, then attend.

    q8: uint8 codes [total_q, Hq, D]; k8: [total_kv, Hkv, D];
    v8_colmajor: [Hkv, D, total_kv] -- V is column-major, i.e. token-contiguous
    for each (head, feature), as [FLEX] _enforce_mem_layouts requires for the
    right operand of ``softmax_scores @ V``.
    descale = (dq, dk, dv): the real tensor is descale * decoded code.
    The result is the exact attention of those real values (fp64).
    """
    dq, dk, dv = (float(x) for x in descale)
    q = dq * e4m3_decode(q8)
    k = dk * e4m3_decode(k8)
    v = dv * np.transpose(e4m3_decode(v8_colmajor), (2, 0, 1))
    return attention_varlen(q, k, v, cu_q, cu_kv, scale, flags, q_ids, kv_ids, rows, window, softcap)
