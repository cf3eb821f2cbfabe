"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws inputs: sequence lengths, block-pool permutations,
patch and document ids, and normally distributed Q/K/V cast to the working
dtype.  It contains none of the attention arithmetic, and it imports neither
the oracle nor the HIP library, so both sides can take identical inputs from
it without sharing code.

Recipe (one ``numpy.random.default_rng(seed)`` for all integer structure, then
one seeded ``torch.Generator`` on the target device for the float tensors):
  1. sequence lengths;
  2. block-pool permutation (sequences take consecutive runs of it);
  3. patch lengths, uniform on {2..14}, drawn until a sequence's bytes are
     covered (cross-attention workload only);
  4. Q, K, V ~ N(0, 1) in float32, in that order, then cast with
     round-to-nearest-even to fp16 / bf16, or for fp8 quantised with a
     per-tensor descale = amax / 448 and cast to float8_e4m3fn.
Unused pool blocks and tail slots are left to the caller to poison (NaN);
unused block_table entries point at a spare pool block so a stray read shows
up as NaN in the output instead of touching memory outside the pool.
"""

from dataclasses import dataclass, field
import math
from typing import Optional

import numpy as np
import torch

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_DOCUMENT = 2
MASK_PATCH = 4

FP8_MAX = 448.0


@dataclass
class Workload:
    name: str
    dtype: str                     # "f16", "bf16" or "fp8"
    q_lens: np.ndarray             # int32 [batch]
    kv_lens: np.ndarray            # int32 [batch]
    new_lens: np.ndarray           # int32 [batch]: tokens written by reshape_and_cache
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    block_table: np.ndarray        # int32 [batch, max_blocks_per_seq]
    mask_flags: int
    scale: float
    q_ids: Optional[np.ndarray] = None    # int32 [total_q] (document id or patch index)
    kv_ids: Optional[np.ndarray] = None   # int32 [total_kv] (document id)
    q: Optional[torch.Tensor] = None      # [total_q, Hq, D]   (decode: [batch, Hq, D])
    k_new: Optional[torch.Tensor] = None  # [total_new, Hkv, D]
    v_new: Optional[torch.Tensor] = None  # [total_new, Hkv, D]
    # fp8 workloads (dense, not paged)
    v8_colmajor: Optional[torch.Tensor] = None  # [Hkv, D, total_kv] uint8 codes
    descale: Optional[np.ndarray] = None        # float32 [3]: dq, dk, dv
    # paged decode over an fp8 cache: k_new / v_new hold uint8 codes
    kv_descale: Optional[np.ndarray] = None     # float32 [2]: dk, dv
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(len(self.q_lens))

    @property
    def total_q(self):
        return int(np.sum(self.q_lens, dtype=np.int64))

    @property
    def total_kv(self):
        return int(np.sum(self.kv_lens, dtype=np.int64))

    @property
    def total_new(self):
        return int(np.sum(self.new_lens, dtype=np.int64))

    @property
    def max_blocks_per_seq(self):
        return int(self.block_table.shape[1])


_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _randn(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _block_table(rng, kv_lens, block_size, pool_blocks=None, spare=True):
    """Random physical placement: sequences take consecutive runs of a permuted pool.

    Returns (block_table int32 [batch, max_blocks], num_blocks).  With
    ``spare`` one extra pool block (never written) fills unused table entries.
    """
    need = [int(math.ceil(int(n) / block_size)) for n in kv_lens]
    used = int(sum(need))
    pool = used if pool_blocks is None else int(pool_blocks)
    if pool < used:
        raise ValueError("pool too small")
    perm = rng.permutation(pool)
    num_blocks = pool + (1 if spare else 0)
    filler = pool if spare else int(perm[-1])
    width = max(1, max(need) if need else 1)
    table = np.full((len(kv_lens), width), filler, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, num_blocks


def _patch_ids(rng, n_bytes, lo=2, hi=14):
    """Patch index of every byte: patch lengths uniform on {lo..hi}, drawn until covered."""
    ids = np.empty(n_bytes, dtype=np.int32)
    pos, pid = 0, 0
    while pos < n_bytes:
        length = int(rng.integers(lo, hi, endpoint=True))
        ids[pos:pos + length] = pid
        pos += length
        pid += 1
    return ids, pid


def _cast(x, dtype):
    return x.to(_TORCH_DT[dtype])


def quantize_e4m3(x):
    """Per-tensor fp8 quantisation: descale = amax / 448, codes = RNE(x / descale)."""
    amax = float(x.abs().max())
    descale = amax / FP8_MAX if amax > 0 else 1.0
    codes = (x / descale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, descale


def make_prefill(name, seed, dtype, q_lens, kv_lens, num_heads, num_kv_heads, head_size,
                 block_size, mask_flags, device="cpu", q_ids=None, kv_ids=None,
                 pool_blocks=None, scale=None, rng=None):
    """Paged varlen prefill: every K/V token of a sequence is new (written by
    reshape_and_cache); q_len may differ from kv_len (cross attention)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    q_lens = np.asarray(q_lens, dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    table, num_blocks = _block_table(rng, kv_lens, block_size, pool_blocks)
    w = Workload(name=name, dtype=dtype, q_lens=q_lens, kv_lens=kv_lens, new_lens=kv_lens.copy(),
                 num_heads=num_heads, num_kv_heads=num_kv_heads, head_size=head_size,
                 block_size=block_size, num_blocks=num_blocks, block_table=table,
                 mask_flags=mask_flags,
                 scale=(1.0 / math.sqrt(head_size)) if scale is None else float(scale),
                 q_ids=q_ids, kv_ids=kv_ids)
    if callable(q_ids):
        w.q_ids = q_ids(rng)
    gen = _generator(seed, device)
    tq, tk = w.total_q, w.total_kv
    w.q = _cast(_randn(gen, (tq, num_heads, head_size), device), dtype)
    w.k_new = _cast(_randn(gen, (tk, num_kv_heads, head_size), device), dtype)
    w.v_new = _cast(_randn(gen, (tk, num_kv_heads, head_size), device), dtype)
    return w


def make_decode(name, seed, dtype, kv_lens, num_heads, num_kv_heads, head_size, block_size,
                device="cpu", rng=None):
    """Paged decode: one query per sequence; the whole cache is written once by
    reshape_and_cache before the query attends to it."""
    rng = np.random.default_rng(seed) if rng is None else rng
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    table, num_blocks = _block_table(rng, kv_lens, block_size)
    batch = len(kv_lens)
    w = Workload(name=name, dtype=dtype, q_lens=np.ones(batch, dtype=np.int32), kv_lens=kv_lens,
                 new_lens=kv_lens.copy(), num_heads=num_heads, num_kv_heads=num_kv_heads,
                 head_size=head_size, block_size=block_size, num_blocks=num_blocks,
                 block_table=table, mask_flags=MASK_NONE, scale=1.0 / math.sqrt(head_size))
    gen = _generator(seed, device)
    w.q = _cast(_randn(gen, (batch, num_heads, head_size), device), dtype)
    tk = w.total_kv
    w.k_new = _cast(_randn(gen, (tk, num_kv_heads, head_size), device), dtype)
    w.v_new = _cast(_randn(gen, (tk, num_kv_heads, head_size), device), dtype)
    return w


def make_fp8(name, seed, q_lens, kv_lens, num_heads, num_kv_heads, head_size, mask_flags,
             device="cpu", q_ids=None, kv_ids=None, scale=None):
    """Dense (not paged) varlen fp8 e4m3 attention inputs; V column-major [Hkv, D, total_kv]."""
    q_lens = np.asarray(q_lens, dtype=np.int32)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    w = Workload(name=name, dtype="fp8", q_lens=q_lens, kv_lens=kv_lens,
                 new_lens=np.zeros_like(kv_lens), num_heads=num_heads,
                 num_kv_heads=num_kv_heads, head_size=head_size, block_size=0, num_blocks=0,
                 block_table=np.zeros((len(q_lens), 1), dtype=np.int32), mask_flags=mask_flags,
                 scale=(1.0 / math.sqrt(head_size)) if scale is None else float(scale),
                 q_ids=q_ids, kv_ids=kv_ids)
    gen = _generator(seed, device)
    tq, tk = w.total_q, w.total_kv
    q = _randn(gen, (tq, num_heads, head_size), device)
    k = _randn(gen, (tk, num_kv_heads, head_size), device)
    v = _randn(gen, (tk, num_kv_heads, head_size), device)
    q8, dq = quantize_e4m3(q)
    k8, dk = quantize_e4m3(k)
    v8, dv = quantize_e4m3(v)
    del q, k, v
    w.q = q8
    w.k_new = k8
    w.v8_colmajor = v8.permute(1, 2, 0).contiguous()
    w.descale = np.asarray([dq, dk, dv], dtype=np.float32)
    return w


def to_fp8_cache(w):
    """Turn a paged workload's new K/V tokens into e4m3 codes with per-tensor
    descales (quantize_e4m3); the query keeps its 16-bit type."""
    k8, dk = quantize_e4m3(w.k_new.float())
    v8, dv = quantize_e4m3(w.v_new.float())
    w.k_new, w.v_new = k8, v8
    w.kv_descale = np.asarray([dk, dv], dtype=np.float32)
    w.name += "_fp8kv"
    return w


def make_dout(seed, w, device=None):
    """Upstream gradient for a workload's output: [total_q, Hq, D] ~ N(0, 1)
    in the workload's 16-bit type."""
    device = w.q.device if device is None else device
    gen = _generator(seed, device)
    return _cast(_randn(gen, (w.total_q, w.num_heads, w.head_size), device), w.dtype)


def rope_tables(max_position, rotary_dim, base=10000.0):
    """Angle tables of the usual rotary embedding, float32 [max_position,
    rotary_dim / 2]: entry (p, j) is cos / sin of p * base^(-2j / rotary_dim)
    (computed in float64, rounded once)."""
    theta = base ** (-np.arange(rotary_dim // 2, dtype=np.float64) * 2.0 / rotary_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_packed_qkv(seed, dtype, total, num_heads, num_kv_heads, head_size, device="cpu"):
    """Packed rows [total, (Hq + 2 Hkv) * D] ~ N(0, 1), cast to dtype."""
    gen = _generator(seed, device)
    return _cast(_randn(gen, (total, (num_heads + 2 * num_kv_heads) * head_size), device), dtype)


def causal_block_mask(q_lens, kv_lens, q_block, kv_block, heads=1):
    """Block lists of a bottom-right causal mask (query i sees key j iff
    j <= i + kv_len - q_len): a key block is full for a query block when the
    block's first row sees its last key, partial when its last row sees its
    first key, hidden otherwise.  Returns int32 arrays kv_num [B, heads, n_qb],
    kv_idx [B, heads, n_qb, n_kb], full_num, full_idx (ids in increasing
    order, zeros past each count)."""
    q_lens, kv_lens = np.asarray(q_lens), np.asarray(kv_lens)
    B = len(q_lens)
    n_qb = max(1, -(-int(q_lens.max(initial=0)) // q_block))
    n_kb = max(1, -(-int(kv_lens.max(initial=0)) // kv_block))
    kv_num = np.zeros((B, heads, n_qb), np.int32)
    kv_idx = np.zeros((B, heads, n_qb, n_kb), np.int32)
    full_num, full_idx = np.zeros_like(kv_num), np.zeros_like(kv_idx)
    for b in range(B):
        ql, kl = int(q_lens[b]), int(kv_lens[b])
        off = kl - ql
        for qb in range(-(-ql // q_block)):
            r0, r1 = qb * q_block, min(ql, (qb + 1) * q_block)
            part, full = [], []
            for kb in range(-(-kl // kv_block)):
                c0, c1 = kb * kv_block, min(kl, (kb + 1) * kv_block)
                if c1 - 1 <= r0 + off:
                    full.append(kb)
                elif c0 <= r1 - 1 + off:
                    part.append(kb)
            kv_num[b, :, qb], full_num[b, :, qb] = len(part), len(full)
            kv_idx[b, :, qb, :len(part)] = part
            full_idx[b, :, qb, :len(full)] = full
    return kv_num, kv_idx, full_num, full_idx


def random_block_mask(rng, q_lens, kv_lens, q_block, kv_block, heads, p_partial=0.4, p_full=0.3,
                      capacity=None, junk=True):
    """Random block lists: each (sequence, head, query block, key block) is
    partial with probability p_partial, else full with p_full, else hidden;
    lists in shuffled order, padded with out-of-range ids (-1, a block past
    the sequence, 10**6) when junk is set."""
    q_lens, kv_lens = np.asarray(q_lens), np.asarray(kv_lens)
    B = len(q_lens)
    n_qb = max(1, -(-int(q_lens.max(initial=0)) // q_block))
    n_kb = max(1, -(-int(kv_lens.max(initial=0)) // kv_block))
    cap = n_kb + 2 if capacity is None else capacity
    kv_num = np.zeros((B, heads, n_qb), np.int32)
    kv_idx = np.zeros((B, heads, n_qb, cap), np.int32)
    full_num, full_idx = np.zeros_like(kv_num), np.zeros_like(kv_idx)
    for b in range(B):
        nk = -(-int(kv_lens[b]) // kv_block)
        for h in range(heads):
            for qb in range(n_qb):
                u = rng.random(nk)
                part = rng.permutation(np.nonzero(u < p_partial)[0])[:cap]
                full = rng.permutation(np.nonzero((u >= p_partial) & (u < p_partial + p_full))[0])[:cap]
                for num, idx, ids in ((kv_num, kv_idx, part), (full_num, full_idx, full)):
                    num[b, h, qb] = len(ids)
                    idx[b, h, qb, :len(ids)] = ids
                    if junk and len(ids) < cap:
                        idx[b, h, qb, len(ids):] = rng.choice([-1, nk, 10 ** 6], cap - len(ids))
    return kv_num, kv_idx, full_num, full_idx


# ---------------------------------------------------------------------------
# The five named workloads and their scaled-down parity variants.
# ---------------------------------------------------------------------------

def tiny_gqa_causal_fp16(device="cpu"):
    """Tiny paged GQA causal prefill, fp16: lens {37, 100}, 4/2 heads, D 64,
    block 16, pages from a permuted pool of 16 blocks (6 unused)."""
    seed = 1001
    rng = np.random.default_rng(seed)
    return make_prefill("tiny_gqa_causal_fp16", seed, "f16", [37, 100], [37, 100], 4, 2, 64, 16,
                        MASK_CAUSAL, device=device, pool_blocks=16, rng=rng)


def varlen_gqa_causal_bf16(device="cpu", batch=16, lo=256, hi=4096, seed=1002):
    """Varlen paged GQA causal prefill, bf16: 16 sequences with lengths uniform
    on [256, 4096], 32/8 heads, D 128, block 16, pool sized to the tokens."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, batch, endpoint=True).astype(np.int32)
    return make_prefill(f"varlen_gqa_causal_bf16_b{batch}_{lo}-{hi}", seed, "bf16", lens, lens,
                        32, 8, 128, 16, MASK_CAUSAL, device=device, rng=rng)


def paged_gqa_decode_bf16(device="cpu", batch=64, lo=1024, hi=32768, seed=1003):
    """Paged GQA decode, bf16: 64 sequences, one query each, KV lengths
    uniform on [1024, 32768], 32/8 heads, D 128, block 16."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, batch, endpoint=True).astype(np.int32)
    return make_decode(f"paged_gqa_decode_bf16_b{batch}_{lo}-{hi}", seed, "bf16", lens, 32, 8,
                       128, 16, device=device, rng=rng)


def paged_gqa_decode_fp8kv(device="cpu", **kw):
    """The paged GQA decode workload above with its K/V cache held as e4m3
    codes (per-tensor descales); bf16 queries and output."""
    return to_fp8_cache(paged_gqa_decode_bf16(device=device, **kw))


def byte_patch_cross_bf16(device="cpu", batch=4, n_bytes=8192, n_keys=1024, seed=1004):
    """Masked byte->patch cross-attention, bf16: 4 sequences of 8192 byte
    queries over 1024 patch keys, 16 heads, D 64; patch lengths uniform on
    {2..14}; a byte sees its own and earlier patches."""
    rng = np.random.default_rng(seed)
    q_lens = np.full(batch, n_bytes, dtype=np.int32)
    kv_lens = np.full(batch, n_keys, dtype=np.int32)
    pool = batch * int(math.ceil(n_keys / 16))

    def ids(r):
        out, counts = [], []
        for _ in range(batch):
            pid, n = _patch_ids(r, n_bytes)
            out.append(pid)
            counts.append(n)
        ids.counts = counts
        return np.concatenate(out).astype(np.int32)

    w = make_prefill(f"byte_patch_cross_bf16_b{batch}_{n_bytes}x{n_keys}", seed, "bf16", q_lens,
                     kv_lens, 16, 16, 64, 16, MASK_PATCH, device=device, q_ids=ids,
                     pool_blocks=pool, rng=rng)
    w.extra["patch_counts"] = ids.counts
    return w


def dense_causal_fp8(device="cpu", batch=4, seqlen=8192, heads=16, seed=1005):
    """Dense causal fp8 e4m3 attention: B 4, H 16, S 8192, D 128, per-tensor
    scales, V column-major, bf16 output."""
    lens = np.full(batch, seqlen, dtype=np.int32)
    return make_fp8(f"dense_causal_fp8_b{batch}_s{seqlen}", seed, lens, lens, heads, heads, 128,
                    MASK_CAUSAL, device=device)
