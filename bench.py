"""Benchmark of the varlen paged GQA attention hot path on one MI355X.

A step is one pass of the prefill hot path over the varlen workload
(16 sequences, lengths uniform on [256, 4096] drawn with seed 1002, 32 query
heads over 8 kv heads, head size 128, block size 16, bf16, causal):
cu_seqlens of the query and kv lengths, reshape_and_cache of every K/V token
into a randomly permuted paged pool, then the fused paged prefill.  Inputs are
resident in HBM before the timed region.  `value` is causal-adjusted
TFLOP/s of the whole step: 4 * D * Hq * sum_b L_b (L_b + 1) / 2 flops (the
visible query-key pairs, each needing a D-long dot product and a D-long
weighted sum) divided by the step time.

The same JSON line carries the prefill kernel's roofline figure (the median
of 50 launches of the prefill alone on the step's inputs, each timed with HIP
events on the launching stream; the mean and median of its launches inside
the timed steps are reported beside it), the fp64 CPU
oracle timed on a bounded sample of the same workload (with the host's CPU
count, the cores this process may use and numpy's BLAS threads) and on
bounded samples of the decode, cross-attention and fp8 workloads, and more
single-GPU
measurements: paged decode (HBM GB/s, with its own roofline figure), the same
decode over an fp8 e4m3 cache (one byte per element), the varlen prefill
under 128x128 causal block lists through the block-sparse entry point, the
fused rotary + packed-QKV unpack + cache write of its tokens (HBM GB/s), a plain
device-to-device copy (the practical HBM ceiling, and the calibration kernel
for the traffic counters), byte->patch cross attention, dense causal fp8 and
the varlen backward on the same workload (TFLOP/s).  The two exp-heavy lines
(cross attention at head size 64, dense fp8) carry a roofline object with
both of their bounds: the MFMA floor and the softmax VALU floor (see
VALU_CYCLES_PER_64), the binding one on top.

`roofline.traffic` is the HBM bytes one prefill launch moves, from the
rocprofv3 FETCH_SIZE / WRITE_SIZE counters recorded in profiles/traffic.json;
it is reported only while the hash of the kernel sources matches the one the
counters were taken with, and is null otherwise.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-extra] [--no-cpu]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Softmax VALU floor (the "alu" bound of the exp-heavy workloads).  From the
# chip's unit counts: 256 CUs x 4 SIMDs at 2.4 GHz; per SIMD a wave-wide
# (64-lane) VALU instruction issues every 4 cycles and v_exp_f32 every 8
# (measured on the box).  Each score needs, per 64 scores: one FMA (scale and
# max shift, 4 cycles), one exp (8), half a v_max3 (2), half a two-value pack
# to the product's type (2), and for the 16-bit kernels one add into the row
# sum (4): 20 cycles, or 16 where the row sum runs on the MFMA (fp8).
# Launches of the prefill alone behind the kernel's roofline figure (median).
KERNEL_LAUNCHES = 50
# Wall time each extra line runs its kernel before it is timed.
WARM_MS = 100.0
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
EXP_PER_S = 64 / 8 * SIMDS * CLOCK_HZ                    # 19.7 T exp/s
VALU_CYCLES_PER_64 = {"bf16": 20.0, "fp8": 16.0}
CSRC = os.path.join(ROOT, "attention_cu_seqlens_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources that define each measured kernel; a change to any of them voids its
# recorded counter traffic
KERNEL_SOURCES = {
    "k_paged_prefill": ["prefill.hip", "ring.h", "device_common.h", "kernels.h"],
    "k_paged_decode": ["decode.hip", "device_common.h", "kernels.h"],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def causal_pairs(q_lens, kv_lens):
    tot = 0
    for ql, kl in zip(q_lens, kv_lens):
        ql, kl = int(ql), int(kl)
        off = kl - ql
        for_rows = np.minimum(np.arange(ql) + off + 1, kl)
        tot += int(np.clip(for_rows, 0, None).sum())
    return tot


def patch_pairs(w):
    cu = np.concatenate([[0], np.cumsum(w.q_lens)])
    tot = 0
    for b in range(w.batch):
        pid = w.q_ids[cu[b]:cu[b + 1]].astype(np.int64)
        tot += int(np.minimum(pid + 1, int(w.kv_lens[b])).sum())
    return tot


def two_bounds(flops, scores, kind, ms, mfma_peak_tflops):
    """Roofline object of an exp-heavy kernel with both of its bounds: the
    MFMA floor (flops at the dense MFMA peak) and the softmax VALU floor
    (scores at the VALU_CYCLES_PER_64 cost), plus the exp floor alone; the
    binding one is the longer floor."""
    mfma_us = flops / (mfma_peak_tflops * 1e12) * 1e6
    valu_per_s = 64 / VALU_CYCLES_PER_64[kind] * SIMDS * CLOCK_HZ
    valu_us = scores / valu_per_s * 1e6
    exp_us = scores / EXP_PER_S * 1e6
    us = ms * 1e3
    tf = flops / (ms * 1e-3) / 1e12
    sc = scores / (ms * 1e-3)
    mfma = {"achieved": round(tf, 2), "peak": mfma_peak_tflops, "unit": "TFLOP/s",
            "frac": round(tf / mfma_peak_tflops, 4), "floor_us": round(mfma_us, 2)}
    valu = {"achieved": round(sc / 1e12, 4), "peak": round(valu_per_s / 1e12, 4),
            "unit": "T scores/s", "frac": round(sc / valu_per_s, 4), "floor_us": round(valu_us, 2),
            "exp_floor_us": round(exp_us, 2), "scores": scores}
    bound = "alu" if valu_us > mfma_us else "mfma"
    top = valu if bound == "alu" else mfma
    return {"bound": bound, "achieved": top["achieved"], "peak": top["peak"],
            "unit": top["unit"], "frac": top["frac"], "kernel_us": round(us, 2),
            "mfma": mfma, "valu": valu}


def warm_up(fn, torch, ms=WARM_MS, max_calls=5000):
    """Runs fn back to back for at least `ms` of wall time before a line is
    timed, so the clocks settle at this kernel's own load: each line follows
    kernels of another kind (an HBM-bound decode before the compute-bound cross
    attention), and a few launches are over before the clocks have moved."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n in range(1, max_calls + 1):
        fn()
        if n % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                break
    torch.cuda.synchronize()


def timed(fn, iters, torch):
    """Median ms per call over `iters` back-to-back calls, each between two
    events on the current stream (the stream the kernels run on)."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def source_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic.json, or None when absent or
    taken with different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[f"{kernel} {workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def i32(a, torch, dev):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32, device=dev)


def paged_inputs(w, A, torch, dev):
    lens_q = i32(w.q_lens, torch, dev)
    lens_kv = i32(w.kv_lens, torch, dev)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_size)
    poison = 0x7F if w.k_new.dtype == torch.uint8 else float("nan")   # NaN (e4m3 code 0x7F)
    kc = torch.full(shape, poison, dtype=w.k_new.dtype, device=dev)
    vc = torch.full(shape, poison, dtype=w.k_new.dtype, device=dev)
    bt = i32(w.block_table, torch, dev)
    return lens_q, lens_kv, kc, vc, bt


def host_threads():
    """Host CPU counts on this machine: (os.cpu_count, cores this process may
    run on, numpy's BLAS thread count -- the threads the oracle's products use)."""
    cpu = os.cpu_count()
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = cpu
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = int(max(blas)) if blas else 1
    except Exception:
        blas_threads = 1
    return cpu, aff, blas_threads


def _contiguous_table(lens, bs):
    """Block table placing the given sequences' pages one after another."""
    nblk = [(int(n) + bs - 1) // bs for n in lens]
    table = np.zeros((len(lens), max(1, max(nblk, default=1))), dtype=np.int32)
    base = 0
    for i, n in enumerate(nblk):
        table[i, :n] = np.arange(base, base + n)
        base += n
    return table, max(1, base)


def _oracle_paged(w, n_seqs, rows_fn=None):
    """The fp64 oracle on the first n_seqs sequences of a paged workload (all
    heads): cache fill through reshape_and_cache, then paged attention (the
    decode form when q_len is 1).  rows_fn(q_lens) may pick sampled rows.
    Returns (seconds, lens_q, lens_kv, rows or None)."""
    import oracle as ORC
    lq = [int(x) for x in w.q_lens[:n_seqs]]
    lk = [int(x) for x in w.kv_lens[:n_seqs]]
    tq, tk = sum(lq), sum(lk)
    q = w.q[:tq].double().cpu().numpy()
    k = w.k_new[:tk].double().cpu().numpy()
    v = w.v_new[:tk].double().cpu().numpy()
    bs = w.block_size
    table, nb = _contiguous_table(lk, bs)
    kc = np.zeros((nb, bs) + k.shape[1:])
    vc = np.zeros_like(kc)
    cu_q, cu_kv = ORC.cu_seqlens(lq), ORC.cu_seqlens(lk)
    rows = None if rows_fn is None else rows_fn(lq)
    ids = None if w.q_ids is None else np.asarray(w.q_ids)[:tq]
    t0 = time.perf_counter()
    kc, vc = ORC.reshape_and_cache(k, v, kc, vc, table, cu_kv, cu_kv, bs)
    ORC.paged_attention(q, kc, vc, table, cu_q, cu_kv, bs, w.scale, w.mask_flags, q_ids=ids,
                        rows=rows)
    return time.perf_counter() - t0, lq, lk, rows


def cpu_baseline(w, n_seqs):
    """The fp64 oracle on the first n_seqs sequences of the varlen prefill
    workload, all heads: cache fill through reshape_and_cache, then paged
    causal attention."""
    cpu, aff, blas = host_threads()
    dt, lens, _, _ = _oracle_paged(w, n_seqs)
    flops = 4.0 * w.head_size * w.num_heads * sum(n * (n + 1) / 2 for n in lens)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "os_cpu_count": cpu, "affinity_cores": aff, "blas_threads": blas,
            "seconds": round(dt, 2),
            "sample": f"sequences 0-{len(lens) - 1} (lengths {lens}) x all {w.num_heads} query "
                      f"heads of the same workload: cache fill + paged causal attention in fp64 "
                      f"numpy, {dt:.1f} s; cores = numpy's BLAS threads (the oracle's products "
                      f"run on them, everything else on one thread)"}


def cpu_baseline_more(W, dev):
    """The fp64 oracle on bounded samples of the decode, cross-attention and
    dense fp8 workloads (CPU only), each reported in its workload's unit."""
    import oracle as ORC
    import torch
    cpu, aff, blas = host_threads()
    res = {}
    log("  oracle: decode sample")
    wd = W.paged_gqa_decode_bf16(device=dev)
    dt, _, lk, _ = _oracle_paged(wd, 6)
    kv_bytes = 2 * sum(lk) * wd.num_kv_heads * wd.head_size * 2
    res["decode"] = {"value": kv_bytes / dt / 1e9, "unit": "GB/s of bf16 K/V", "seconds": round(dt, 2),
                     "sample": f"sequences 0-5 (kv lengths {lk}) x all {wd.num_heads} heads: cache "
                               f"fill + decode in fp64 numpy"}
    del wd
    torch.cuda.empty_cache()
    log(f"  oracle: decode {dt:.1f} s; cross-attention sample")
    wc = W.byte_patch_cross_bf16(device="cpu")
    dt, lq, _, _ = _oracle_paged(wc, 1)
    pid = np.asarray(wc.q_ids)[:lq[0]].astype(np.int64)
    pairs = int(np.minimum(pid + 1, int(wc.kv_lens[0])).sum())
    res["cross_attention"] = {
        "value": 4.0 * wc.head_size * wc.num_heads * pairs / dt / 1e12, "unit": "TFLOP/s",
        "seconds": round(dt, 2), "sample": f"sequence 0 (8192 bytes x 1024 patch keys) x all "
                                           f"{wc.num_heads} heads"}
    del wc
    log(f"  oracle: cross {dt:.1f} s; fp8 sample")
    w8 = W.dense_causal_fp8(device="cpu", batch=1)
    stride = 512
    rows = np.arange(0, int(w8.q_lens[0]), stride)
    cu = ORC.cu_seqlens(w8.q_lens)
    t0 = time.perf_counter()
    ORC.fp8_attention(w8.q.numpy(), w8.k_new.numpy(), w8.v8_colmajor.numpy(), w8.descale, cu, cu,
                      w8.scale, w8.mask_flags, rows=rows)
    dt = time.perf_counter() - t0
    pairs = int((rows + 1).sum())
    res["fp8"] = {"value": 4.0 * w8.head_size * w8.num_heads * pairs / dt / 1e12,
                  "unit": "TFLOP/s", "seconds": round(dt, 2),
                  "sample": f"every {stride}th query row of sequence 0 (of 8192) x all "
                            f"{w8.num_heads} heads, causal"}
    del w8
    log(f"  oracle: fp8 {dt:.1f} s")
    for r in res.values():
        r.update({"kind": "oracle", "cores": blas})
    res["host"] = {"os_cpu_count": cpu, "affinity_cores": aff, "blas_threads": blas}
    return res


def bench_copy(torch, dev, nbytes=2 << 30, iters=20):
    """Device-to-device copy: the practical HBM ceiling (read + write bytes)."""
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    warm_up(lambda: y.copy_(x), torch)
    ms = timed(lambda: y.copy_(x), iters, torch)
    del x, y
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"bytes_copied": nbytes, "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def bench_decode(A, W, torch, dev, iters=50, fp8kv=False):
    """Paged GQA decode; with fp8kv the cache holds e4m3 codes (one byte per
    element, per-tensor descales) and the fp8-cache entry point runs."""
    w = W.paged_gqa_decode_fp8kv(device=dev) if fp8kv else W.paged_gqa_decode_bf16(device=dev)
    lens_q, lens_kv, kc, vc, bt = paged_inputs(w, A, torch, dev)
    cu_kv = A.attn_cu_seqlens(lens_kv)
    A.attn_reshape_and_cache(w.k_new, w.v_new, kc, vc, bt, cu_kv, cu_kv)
    elem = w.k_new.element_size()
    del w.k_new, w.v_new
    maxkv = int(w.kv_lens.max())
    need = A.attn_paged_decode_workspace_bytes(w.batch, w.num_heads, w.num_kv_heads, w.head_size,
                                               maxkv)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty_like(w.q)
    if fp8kv:
        ds = torch.as_tensor(w.kv_descale, dtype=torch.float32).to(dev)

        def run():
            A.attn_paged_decode_fp8kv_fwd(w.q, kc, vc, ds, bt, cu_kv, maxkv, scale=w.scale,
                                          out=out, workspace=ws)
    else:
        def run():
            A.attn_paged_decode_fwd(w.q, kc, vc, bt, cu_kv, maxkv, scale=w.scale, out=out,
                                    workspace=ws)

    warm_up(run, torch)
    ms = timed(run, iters, torch)
    tokens = int(w.kv_lens.sum())
    used_blocks = int(sum(math.ceil(int(n) / w.block_size) for n in w.kv_lens))
    nbytes = (2 * tokens * w.num_kv_heads * w.head_size * elem + 2 * w.q.numel() * 2
              + used_blocks * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": w.name, "ms": round(ms, 4), "GB/s": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
           "roofline": {"kernel": "k_paged_decode + k_decode_combine", "bound": "hbm",
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": recorded_traffic("k_paged_decode", w.name)}}
    del kc, vc
    torch.cuda.empty_cache()
    return res


def bench_rotary_cache(A, W, torch, dev, iters=50):
    """Rotary + packed-QKV unpack + cache write of the varlen workload's
    34,805 tokens (bf16, 32 + 2 x 8 heads, D 128, full-width rotary): HBM
    bytes = the packed rows read + q_out, K and V written + the angle-table
    rows read."""
    w = W.varlen_gqa_causal_bf16(device=dev)
    lens_q, lens_kv, kc, vc, bt = paged_inputs(w, A, torch, dev)
    cu = A.attn_cu_seqlens(lens_kv)
    total, hq, hkv, d = w.total_q, w.num_heads, w.num_kv_heads, w.head_size
    del w.k_new, w.v_new, w.q
    qkv = W.make_packed_qkv(1006, "bf16", total, hq, hkv, d, device=dev)
    cos, sin = (torch.from_numpy(t).to(dev) for t in W.rope_tables(int(w.kv_lens.max()), d))
    q_out = torch.empty((total, hq, d), dtype=torch.bfloat16, device=dev)
    maxkv = int(w.kv_lens.max())

    def run():
        A.attn_rotary_reshape_and_cache(kc, vc, bt, cu, cu, maxkv, qkv=qkv, num_heads=hq,
                                        cos_table=cos, sin_table=sin, q_out=q_out)

    warm_up(run, torch)
    ms = timed(run, iters, torch)
    nbytes = 2 * qkv.numel() * 2 + total * d * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": w.name + "_packed_qkv_rotary", "ms": round(ms, 4), "GB/s": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes}
    del kc, vc, qkv, q_out
    torch.cuda.empty_cache()
    return res


def bench_prefill_generic(A, W, torch, dev, w, flops, iters=50, block_mask=None):
    """Paged prefill of w; block_mask = (q_block, kv_block, kv_num, kv_idx,
    full_num, full_idx) numpy arrays runs the block-sparse entry point."""
    lens_q, lens_kv, kc, vc, bt = paged_inputs(w, A, torch, dev)
    cu_q = A.attn_cu_seqlens(lens_q)
    cu_kv = A.attn_cu_seqlens(lens_kv)
    A.attn_reshape_and_cache(w.k_new, w.v_new, kc, vc, bt, cu_kv, cu_kv)
    q_ids = None if w.q_ids is None else i32(w.q_ids, torch, dev)
    out = torch.empty_like(w.q)
    if block_mask is not None:
        qbs, kbs, *lists = block_mask
        kn, ki, fn, fi = (i32(a, torch, dev) for a in lists)

        def run():
            A.attn_paged_prefill_block_sparse_fwd(
                w.q, kc, vc, bt, cu_q, cu_kv, int(w.q_lens.max()), int(w.kv_lens.max()), qbs, kbs,
                kn, ki, fn, fi, scale=w.scale, mask_flags=w.mask_flags, q_ids=q_ids, out=out)
    else:
        def run():
            A.attn_paged_prefill_fwd(w.q, kc, vc, bt, cu_q, cu_kv, int(w.q_lens.max()),
                                     int(w.kv_lens.max()), scale=w.scale, mask_flags=w.mask_flags,
                                     q_ids=q_ids, out=out)

    warm_up(run, torch)
    ms = timed(run, iters, torch)
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops": flops}


def bench_backward(A, W, torch, dev, iters=20):
    """Varlen backward (dQ with the row sums delta, then dK/dV) on the varlen causal
    workload, packed K / V; O and the LSE from the paged forward.  Work is
    counted the usual way, 2.5x the forward's causal flops (five products
    per visible pair: S, dP, dV, dK, dQ); the kernels recompute S and dP in
    both the dQ and the dK/dV pass, seven products in all."""
    w = W.varlen_gqa_causal_bf16(device=dev)
    lens_q, lens_kv, kc, vc, bt = paged_inputs(w, A, torch, dev)
    cu_q = A.attn_cu_seqlens(lens_q)
    cu_kv = A.attn_cu_seqlens(lens_kv)
    A.attn_reshape_and_cache(w.k_new, w.v_new, kc, vc, bt, cu_kv, cu_kv)
    mq, mk = int(w.q_lens.max()), int(w.kv_lens.max())
    out, lse = A.attn_paged_prefill_fwd(w.q, kc, vc, bt, cu_q, cu_kv, mq, mk, scale=w.scale,
                                        mask_flags=w.mask_flags, return_lse=True)
    del kc, vc
    dout = W.make_dout(1007, w)
    dq, dk, dv = torch.empty_like(w.q), torch.empty_like(w.k_new), torch.empty_like(w.v_new)
    ws = torch.empty(A.attn_varlen_bwd_workspace_bytes(w.total_q, w.num_heads), dtype=torch.uint8,
                     device=dev)

    def run():
        A.attn_varlen_bwd(w.q, w.k_new, w.v_new, out, dout, lse, cu_q, cu_kv, mq, mk,
                          scale=w.scale, mask_flags=w.mask_flags, dq=dq, dk=dk, dv=dv,
                          workspace=ws)

    warm_up(run, torch)
    ms = timed(run, iters, torch)
    flops = 2.5 * 4.0 * w.head_size * w.num_heads * causal_pairs(w.q_lens, w.kv_lens)
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": w.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
           "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops": flops,
           "flops_convention": "2.5 x forward causal flops"}
    del out, lse, dout, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def bench_fp8(A, W, torch, dev, iters=50):
    w = W.dense_causal_fp8(device=dev)
    cu_q = A.attn_cu_seqlens(i32(w.q_lens, torch, dev))
    ds = torch.as_tensor(w.descale, dtype=torch.float32, device=dev)
    out = torch.empty((w.total_q, w.num_heads, w.head_size), dtype=torch.bfloat16, device=dev)
    flops = 4.0 * w.head_size * w.num_heads * causal_pairs(w.q_lens, w.kv_lens)

    def run():
        A.attn_fp8_fwd(w.q, w.k_new, w.v8_colmajor, ds, cu_q, cu_q, int(w.q_lens.max()),
                       int(w.kv_lens.max()), scale=w.scale, mask_flags=w.mask_flags, out=out)

    warm_up(run, torch)
    ms = timed(run, iters, torch)
    tf = flops / (ms * 1e-3) / 1e12
    scores = causal_pairs(w.q_lens, w.kv_lens) * w.num_heads
    return {"workload": w.name, "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
            "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4), "flops": flops,
            "roofline": two_bounds(flops, scores, "fp8", ms, PEAK_FP8_TFLOPS)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip decode / cross / fp8 lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seqs", type=int, default=3,
                    help="sequences of the workload in the CPU oracle sample")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this attention hot path has no multi-GPU "
              "code (each GPU would run its own heads or sequences); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_cu_seqlens_amd as A
    import workloads as W

    A._lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating the varlen prefill workload")
    w = W.varlen_gqa_causal_bf16(device=dev)
    lens_q, lens_kv, kc, vc, bt = paged_inputs(w, A, torch, dev)
    cu_q = torch.empty(w.batch + 1, dtype=torch.int32, device=dev)
    cu_kv = torch.empty(w.batch + 1, dtype=torch.int32, device=dev)
    out = torch.empty_like(w.q)
    max_q, max_kv = int(w.q_lens.max()), int(w.kv_lens.max())
    pairs = causal_pairs(w.q_lens, w.kv_lens)
    flops = 4.0 * w.head_size * w.num_heads * pairs
    stream = torch.cuda.current_stream()
    k_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]

    def step(i=None):
        A.attn_cu_seqlens(lens_q, out=cu_q)
        A.attn_cu_seqlens(lens_kv, out=cu_kv)
        A.attn_reshape_and_cache(w.k_new, w.v_new, kc, vc, bt, cu_kv, cu_kv)
        if i is not None:
            k_ev[i][0].record(stream)
        A.attn_paged_prefill_fwd(w.q, kc, vc, bt, cu_q, cu_kv, max_q, max_kv, scale=w.scale,
                                 mask_flags=w.mask_flags, out=out)
        if i is not None:
            k_ev[i][1].record(stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    k_all = [a.elapsed_time(b) for a, b in k_ev]
    value = flops / (ms_step * 1e-3) / 1e12
    # The kernel's roofline figure: the median of KERNEL_LAUNCHES launches of
    # the prefill alone on the same inputs (cache filled by the steps above),
    # each between two events on the launching stream.
    iso = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(KERNEL_LAUNCHES)]
    for a, b in iso:
        a.record(stream)
        A.attn_paged_prefill_fwd(w.q, kc, vc, bt, cu_q, cu_kv, max_q, max_kv, scale=w.scale,
                                 mask_flags=w.mask_flags, out=out)
        b.record(stream)
    torch.cuda.synchronize()
    k_iso = [a.elapsed_time(b) for a, b in iso]
    k_med = float(np.median(k_iso))
    achieved = flops / (k_med * 1e-3) / 1e12
    log(f"step {ms_step:.4f} ms (wall {wall * 1e3 / args.steps:.4f} ms), prefill kernel "
        f"{k_med:.4f} ms (median of {KERNEL_LAUNCHES}), {np.mean(k_all):.4f} ms inside the steps")

    line = {
        "metric": "prefill attn TFLOP/s (causal-adjusted) + decode HBM GB/s, % of MI355X peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "total_tokens": w.total_q,
                   "max_seqlen": max_q, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size, "mask": "causal", "seed": 1002,
                   "step": "cu_seqlens x2 + reshape_and_cache + paged prefill",
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "k_paged_prefill", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("k_paged_prefill", w.name),
                     "kernel_ms": round(k_med, 5), "kernel_ms_mean": round(float(np.mean(k_iso)), 5),
                     "launches": KERNEL_LAUNCHES,
                     "kernel_ms_in_steps_mean": round(float(np.mean(k_all)), 5),
                     "kernel_ms_in_steps_median": round(float(np.median(k_all)), 5),
                     "flops_per_launch": flops},
    }
    del kc, vc, out
    torch.cuda.empty_cache()

    if not args.no_extra:
        log("hbm copy")
        line["hbm_copy"] = bench_copy(torch, dev)
        log("decode")
        line["decode"] = bench_decode(A, W, torch, dev)
        torch.cuda.empty_cache()
        log("decode, fp8 cache")
        line["decode_fp8kv"] = bench_decode(A, W, torch, dev, fp8kv=True)
        torch.cuda.empty_cache()
        log("byte->patch cross attention")
        wc = W.byte_patch_cross_bf16(device=dev)
        pp = patch_pairs(wc)
        line["cross_attention"] = bench_prefill_generic(
            A, W, torch, dev, wc, 4.0 * wc.head_size * wc.num_heads * pp)
        line["cross_attention"]["roofline"] = two_bounds(
            line["cross_attention"]["flops"], pp * wc.num_heads, "bf16",
            line["cross_attention"]["ms"], PEAK_BF16_TFLOPS)
        del wc
        torch.cuda.empty_cache()
        log("rotary + packed-QKV unpack + cache write")
        line["rotary_cache"] = bench_rotary_cache(A, W, torch, dev)
        log("block-sparse prefill, causal block lists")
        wb = W.varlen_gqa_causal_bf16(device=dev)
        bm = (128, 128) + W.causal_block_mask(wb.q_lens, wb.kv_lens, 128, 128)
        line["block_sparse"] = bench_prefill_generic(
            A, W, torch, dev, wb, 4.0 * wb.head_size * wb.num_heads
            * causal_pairs(wb.q_lens, wb.kv_lens), block_mask=bm)
        line["block_sparse"]["blocks"] = "128x128 FlexAttention-style causal lists"
        del wb
        torch.cuda.empty_cache()
        log("fp8")
        line["fp8"] = bench_fp8(A, W, torch, dev)
        log("varlen backward")
        line["backward"] = bench_backward(A, W, torch, dev)

    if not args.no_cpu:
        log("cpu oracle baseline")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seqs)
        if not args.no_extra:
            log("cpu oracle baselines of the decode, cross and fp8 workloads")
            line["cpu_baseline_other_workloads"] = cpu_baseline_more(W, dev)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
