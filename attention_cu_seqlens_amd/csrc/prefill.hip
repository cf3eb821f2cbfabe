// Paged varlen GQA prefill for 16-bit dtypes on gfx950.
//
// One workgroup owns a tile of BM packed query rows and runs the whole key
// range they can see: online softmax over BN-key tiles of the paged cache
// (the fused form of the gather + varlen attention path of the onnxruntime
// PR "[CUDA] PagedAttention: add SM<80 fp16 fallback via memory-efficient
// attention", section Implementation, steps 2-3).
//
// Row packing: the P = 2^pack_log2 query heads of one workgroup share a kv
// head (GQA); packed row r is token r >> pack_log2, head h0 + (r & (P-1)).
// Every K/V tile staged in LDS therefore serves P heads, and the causal
// diagonal of a tile spans BM / P tokens.
//
// Work decomposition needs no device->host sync: the host bounds the grid by
// max_seqlen_q and total_q, and each workgroup finds its (sequence, head
// group, query tile) from cu_seqlens_q (map_tile); the few workgroups past
// the last tile exit at once.
//
// Masks reduce to one visible key interval [lo, hi) per query row: causal
// (bottom-right) and patch bound hi, document ids (non-decreasing within a
// sequence) bound both.  Each wave classifies every key tile as empty (skip),
// full (no per-element test) or partial from the extreme intervals of its
// rows.

#include "device_common.h"
#include "kernels.h"
#include "ring.h"

namespace attn {

// Ring depth: up to kStages - 1 tiles in flight while one is consumed.
constexpr int kStages = 4;

// Per-wave pipeline state of one 32-row block.
template <int D, int BN>
struct PrefillWave {
    static constexpr int NPRE = pv_preload<D, BN>();
    f32x16_t s[BN / 32];      // scores of the tile waiting for its softmax
    u32x4_t pb[BN / 32][2];   // probabilities of the tile waiting for its P.V
    u32x4_t pre[NPRE > 0 ? NPRE : 1];   // first V^T operands of that P.V, read ahead
    f32x16_t o[D / 32];
    float m, lpart, alpha;
    bool need;
};

// Softmax phase (VALU): mask the scores of the tile at key j0 when partial,
// then probabilities into pb (scores capped first with CAP); finally read
// the first operands of the tile's P.V from its V tile v_tile.
template <int D, int BN, bool BF16, bool CAP>
__device__ __forceinline__ void phase_softmax(PrefillWave<D, BN>& st, bool partial, int j0, int lo,
                                              int hi, float c, const uint8_t* v_tile,
                                              float cap_in2, float cap_out) {
    if (partial) {
        const int g = lane_id() >> 5;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (!(key >= lo && key < hi)) st.s[kb][r] = kNegInf;
            }
        softmax_tile<BN, BF16, true, CAP>(st.s, c, st.m, st.lpart, st.pb, st.alpha, st.need,
                                          cap_in2, cap_out);
    } else {
        softmax_tile<BN, BF16, false, CAP>(st.s, c, st.m, st.lpart, st.pb, st.alpha, st.need,
                                           cap_in2, cap_out);
    }
    preload_pv<D, BN, PrefillWave<D, BN>::NPRE>(st.pre, v_tile);
}

// The MFMA work of a phase: P.V of the softmaxed tile (after the rare
// rescale; `hook` runs after each of its MFMAs) when PV, then QK of the next
// tile when QK.
template <int D, int BN, bool BF16, bool PV, bool QK, class Hook = NoHook>
__device__ __forceinline__ void step_mfma(PrefillWave<D, BN>& st, const u32x4_t (&q)[D / 16],
                                          const uint8_t* v_tile, const uint8_t* k_tile,
                                          const Hook& hook = Hook{}) {
    if (PV && st.need) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) st.o[db] *= st.alpha;
        st.need = false;
    }
    // The MFMA phase runs at raised wave priority: when both waves of a SIMD
    // are ready, its LDS reads and MFMAs issue ahead of the other wave's
    // softmax VALU work (+1.7% on the varlen workload, output unchanged).
    __builtin_amdgcn_s_setprio(1);
    mfma_stream16<D, BN, BF16, PV, QK, PrefillWave<D, BN>::NPRE>(st.o, st.s, st.pb, q, st.pre,
                                                                v_tile, k_tile, hook);
    __builtin_amdgcn_s_setprio(0);
}

template <int D, int BN, int QB, int NW, bool BF16, bool CAP, bool BSP>
__global__ __launch_bounds__(NW * 64) void k_paged_prefill(PrefillParams p) {
    static_assert(QB == 1 && NW == 8, "two groups of four single-block waves");
    constexpr int BM = NW * 32;
    static_assert(BM == kPrefillRows, "rows per workgroup as the host assumes");
    static_assert(PAGE_WIN * 64 / BN <= NW * 64, "a chunk's tiles fit one per thread");
    using R = Ring16<D, BN, NW / 2>;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages * R::STAGE];
    __shared__ int wave_range[2][NW];
    __shared__ int win[PAGE_WIN + 1];
    // Stored block-sparse mask: the state of every key block for each query
    // block the workgroup's rows touch (0 hidden, 1 partial, 2 full), and per
    // key chunk the list of its tiles that some query block lists.
    __shared__ uint32_t bstate[BSP ? kBlockStateBytes / 4 : 1];
    __shared__ uint16_t tlist[BSP ? NW * 64 : 1];
    __shared__ int bsum[NW + 2];
    __shared__ int bcnt[BSP ? 16 : 1];
    const uint8_t* bstate8 = reinterpret_cast<const uint8_t*>(bstate);

    int b, hg, qt;
    if (!map_tile(p.cu_q, p.batch, p.n_head_groups, BM >> p.pack_log2, blockIdx.x & 7,
                  blockIdx.x >> 3, b, hg, qt))
        return;

    const int q_start = p.cu_q[b];
    const int q_len = p.cu_q[b + 1] - q_start;
    const int tok0 = qt * (BM >> p.pack_log2);
    const int kv_start = p.cu_kv[b];
    const int kv_len = p.cu_kv[b + 1] - kv_start;
    const int h0 = hg << p.pack_log2;
    const int hk = h0 / p.group;
    const bool neg = p.c < 0.f;
    const float c = fabsf(p.c);

    const int tid = threadIdx.x;
    // Block-sparse set-up, first half: the list counts of the query blocks
    // this workgroup touches are loaded here, so their latency overlaps the
    // Q loads and interval searches below; the state words are cleared.
    int bm_cnt = 0;
    int n_lq = 1, qb0 = 0, mh = 0;
    if constexpr (BSP) {
        n_lq = max(1, (BM >> p.pack_log2) >> p.bm_qbs_log2);   // at most 8
        qb0 = tok0 >> p.bm_qbs_log2;
        mh = p.bm_heads == 1 ? 0 : (p.bm_heads == p.num_heads ? h0 : hk);
        const int qb_last = q_len > 0 ? (q_len - 1) >> p.bm_qbs_log2 : -1;
        if (tid < 2 * n_lq) {
            const int pass = tid >= n_lq, qb = qb0 + tid - pass * n_lq;
            const int32_t* num = pass ? p.bm_full_num : p.bm_kv_num;
            if (num != nullptr && qb <= qb_last && qb < p.bm_nqb)
                bm_cnt = min(max(num[((int64_t)b * p.bm_heads + mh) * p.bm_nqb + qb], 0), p.bm_cap);
        }
        for (int i = tid; i < (n_lq * p.bm_n_kb + 3) / 4; i += NW * 64) bstate[i] = 0u;
        if (tid == 0) {
            bsum[NW] = 0x7fffffff;
            bsum[NW + 1] = -1;
        }
    }
    const int lane = lane_id();
    const int w = wave_id();
    const int col = lane & 31, g = lane >> 5;
    // Waves 0-3 and 4-7 each hold one wave per SIMD; the second group runs
    // half a tile behind the first, so on every SIMD one wave issues MFMAs
    // while the other computes a softmax.  The first group alone loads the
    // K/V ring, between the MFMAs of its MFMA phase.
    const bool lead = w < NW / 2;

    // this lane's query row
    const int r = w * 32 + col;
    const int tok = tok0 + (r >> p.pack_log2);
    const int head = h0 + (r & ((1 << p.pack_log2) - 1));
    const bool valid = tok < q_len;
    // Q operand; a row past the sequence end reads row tok0 instead (its keys
    // are all masked and it is never stored), so the loads issue back to back
    // with no branch and their latency overlaps the set-up below.
    u32x4_t q[D / 16];
    {
        const uint16_t* qp =
            p.q + ((int64_t)(q_start + (valid ? tok : tok0)) * p.num_heads + head) * D + 8 * g;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) q[t] = *reinterpret_cast<const u32x4_t*>(qp + 16 * t);
        if (neg) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) q[t] = neg16x8(q[t]);
        }
    }
    int lo = 0, hi = 0;
    if (valid) {
        hi = kv_len;
        if (p.mask & kMaskCausal) hi = min(hi, tok + (kv_len - q_len) + 1);
        if (p.mask & kMaskPatch) hi = min(hi, p.q_ids[q_start + tok] + 1);
        if (p.mask & kMaskDocument) {
            const int doc = p.q_ids[q_start + tok];
            lo = lower_bound_i32(p.kv_ids + kv_start, kv_len, doc);
            hi = min(hi, upper_bound_i32(p.kv_ids + kv_start, kv_len, doc));
        }
        // local window: keys after the query's own position minus the window
        if (p.window > 0) lo = max(lo, tok + (kv_len - q_len) - p.window + 1);
        if (hi < lo) hi = lo;
    }
    // Wave extremes over valid rows; an all-invalid wave gets an empty range.
    const int w_lo = wave_min(valid ? lo : 0x7fffffff);
    const int w_hi = wave_max(valid ? hi : -0x7fffffff);
    const int w_lo_max = wave_max(valid ? lo : -0x7fffffff);
    const int w_hi_min = wave_min(valid ? hi : 0x7fffffff);
    const bool w_any = w_hi > w_lo;
    if (lane == 0) {
        wave_range[0][w] = w_any ? w_lo : 0x7fffffff;
        wave_range[1][w] = w_any ? w_hi : -0x7fffffff;
    }
    if (BSP && tid < 2 * n_lq) bcnt[tid] = bm_cnt;
    __syncthreads();
    int kv_begin = 0x7fffffff, kv_end = -0x7fffffff;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        kv_begin = min(kv_begin, wave_range[0][i]);
        kv_end = max(kv_end, wave_range[1][i]);
    }
    kv_begin &= ~15;

    // The element mask's key range, [el_lo, el_hi): a partial block's tiles
    // outside it hold no visible key for any row of the workgroup.
    const int el_lo = kv_begin, el_hi = kv_end;

    // Block-sparse set-up, second half: read the listed block ids (flattened
    // over the 2 * n_lq lists) and set their state bits, bit 0 partial and
    // bit 1 full, one byte per (local query block, key block); a block in
    // both lists reads as full.  This wave's rows lie in one query block
    // (its 32 >> pack tokens are aligned and a query block holds at least
    // 32 tokens).  The key range becomes that of the listed blocks.
    int lq_w = 0;
    if constexpr (BSP) {
        const int n_kb = p.bm_n_kb;
        lq_w = ((tok0 + ((w * 32) >> p.pack_log2)) >> p.bm_qbs_log2) - qb0;
        // key blocks of this sequence that have a state byte (a kv_len above
        // max_seqlen_kv would otherwise run past the row)
        const int n_kb_seq = min(n_kb, kv_len > 0 ? ((kv_len - 1) >> p.bm_kvbs_log2) + 1 : 0);
        int total = 0;
        for (int k = 0; k < 2 * n_lq; ++k) total += bcnt[k];
        for (int e = tid; e < total; e += NW * 64) {
            int k = 0, base = 0;
            while (e >= base + bcnt[k]) base += bcnt[k++];
            const int pass = k >= n_lq, lq = k - pass * n_lq;
            const int32_t* idx = pass ? p.bm_full_idx : p.bm_kv_idx;
            const int64_t row = ((int64_t)b * p.bm_heads + mh) * p.bm_nqb + qb0 + lq;
            const int kb = idx[row * p.bm_cap + (e - base)];
            if (kb >= 0 && kb < n_kb_seq) {
                const int at = lq * n_kb + kb;
                atomicOr(&bstate[at >> 2], (pass ? 2u : 1u) << (8 * (at & 3)));
                atomicMin(&bsum[NW], kb);
                atomicMax(&bsum[NW + 1], kb);
            }
        }
        __syncthreads();
        const int kb_lo = bsum[NW], kb_hi = bsum[NW + 1];
        if (kb_hi < kb_lo) {
            kv_begin = kv_end = 0;
        } else {
            kv_begin = kb_lo << p.bm_kvbs_log2;
            kv_end = (int)min((int64_t)kv_len, (int64_t)(kb_hi + 1) << p.bm_kvbs_log2);
        }
    }
    kv_begin = __builtin_amdgcn_readfirstlane(kv_begin);
    kv_end = __builtin_amdgcn_readfirstlane(kv_end);

    const int32_t* table = p.block_table + (int64_t)b * p.mbps;
    const int n_blocks = (kv_len + (1 << p.bs_log2) - 1) >> p.bs_log2;
    const int tok_stride = p.num_kv_heads * D;
    const int head_off = hk * D;
    const int chunk_keys = PAGE_WIN << p.bs_log2;   // a multiple of BN
    R ld;
    ld.init(lane, w & (NW / 2 - 1), tok_stride);
    const uint32_t ring_lds = lds_addr(ring);

    PrefillWave<D, BN> st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16_t{};
    st.m = kNegInf;
    st.lpart = 0.f;
    st.alpha = 1.f;
    st.need = false;

    // Key chunks of PAGE_WIN blocks: stage the chunk's block ids, then stream
    // its tiles through the ring.
    //
    // Per tile j each wave runs QK(j) -> softmax(j) -> PV(j).  The two waves
    // of a SIMD are offset by half a tile, so that one issues MFMAs (and their
    // LDS operand reads) while the other runs the softmax on the VALU:
    //   phase 1 of tile j: lead softmax(j)               trail PV(j-1), QK(j)
    //   phase 2 of tile j: lead PV(j), QK(j+1), loads    trail softmax(j)
    // The lead waves alone load the ring: tile j+3 goes into the stage of
    // tile j-1 (free once phase 1 of tile j is over), one load after every
    // other MFMA of the lead's P.V.
    // The trailing waves' first P.V of a chunk multiplies P = 0 (pb zeroed
    // here and after each chunk) by the V tile of the last stage: zeroed here
    // (uninitialised LDS could hold NaN codes), later a finite cache tile.
    constexpr int kPvSteps = (D / 32) * (BN / 32) * 2;
    static_assert(kPvSteps % R::LOADS_PER_TILE == 0, "loads spread evenly over the MFMAs");
    using Hook = DmaHook<R, kPvSteps / R::LOADS_PER_TILE>;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) st.pb[kb][0] = st.pb[kb][1] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < (PrefillWave<D, BN>::NPRE > 0 ? PrefillWave<D, BN>::NPRE : 1); ++i)
        st.pre[i] = u32x4_t{0u, 0u, 0u, 0u};
    for (int i = tid; i < R::TILE / 16; i += NW * 64)
        *reinterpret_cast<u32x4_t*>(ring + (kStages - 1) * R::STAGE + R::TILE + 16 * i) =
            u32x4_t{0u, 0u, 0u, 0u};
    for (int cs = kv_begin; cs < kv_end; cs += chunk_keys) {
        int n = (min(kv_end, cs + chunk_keys) - cs + BN - 1) / BN;
        const int first = cs >> p.bs_log2;
        fill_page_window(win, table, first, n_blocks, tid, NW * 64);
        if constexpr (BSP) {
            // compact the chunk's listed tiles (thread t looks at tile t)
            bool on = false;
            if (tid < n) {
                const int jt = cs + tid * BN;
                const int kb = jt >> p.bm_kvbs_log2;
                int v = 0;
                for (int lq = 0; lq < n_lq; ++lq) v |= bstate8[lq * p.bm_n_kb + kb];
                on = (v & 2) || ((v & 1) && jt < el_hi && jt + BN > el_lo);
            }
            const uint64_t bal = __ballot(on);
            if (lane == 0) bsum[w] = __popcll(bal);
            __syncthreads();
            int off = 0, tot = 0;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                off += i < w ? bsum[i] : 0;
                tot += bsum[i];
            }
            if (on) tlist[off + __popcll(bal & ((1ull << lane) - 1))] = (uint16_t)tid;
            n = tot;
        }
        __syncthreads();
        // key offset of the chunk's k-th tile (listed tiles only when sparse)
        auto tile_key = [&](int k) {
            if constexpr (BSP) return cs + (int)tlist[max(0, min(k, n - 1))] * BN;
            else return cs + k * BN;
        };
        if (lead) {
#pragma unroll
            for (int k = 0; k < kStages - 1; ++k)
                if (k < n) {
                    const int jk = tile_key(k);
                    ld.issue(ring_lds + k * R::STAGE, p.k_cache, p.v_cache, win, first, jk,
                             kv_len, p.bs_log2, tok_stride, head_off, w,
                             win[R::slot(jk, first, p.bs_log2, w)]);
                }
            // tile 0 must have landed; tiles 1 and 2 may stay in flight
            static_assert(kStages == 4, "wait counts below");
            if (n > 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * R::LOADS_PER_TILE));
            else if (n > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::LOADS_PER_TILE));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        block_barrier();
        if (lead) step_mfma<D, BN, BF16, false, true>(st, q, ring, ring);

        for (int jt = 0; jt < n; ++jt) {
            const int j0 = tile_key(jt);
            bool partial = !(w_any && j0 >= w_lo_max && j0 + BN <= w_hi_min);
            int lo_t = lo, hi_t = hi;   // this tile's visible interval per row
            if constexpr (BSP) {
                const int v = __builtin_amdgcn_readfirstlane(
                    bstate8[lq_w * p.bm_n_kb + (j0 >> p.bm_kvbs_log2)]);
                const int stt = v >= 2 ? 2 : v;
                if (stt == 2) {          // full block: every existing key
                    lo_t = 0;
                    hi_t = valid ? kv_len : 0;
                    partial = j0 + BN > kv_len;
                } else if (stt == 0) {   // not listed for this wave's rows
                    lo_t = hi_t = 0;
                    partial = true;
                }
            }
            const uint8_t* st_cur = ring + (jt % kStages) * R::STAGE;
            const uint8_t* st_prev = ring + ((jt + kStages - 1) % kStages) * R::STAGE;
            const uint8_t* st_next = ring + ((jt + 1) % kStages) * R::STAGE;
            // phase 1
            if (lead)
                phase_softmax<D, BN, BF16, CAP>(st, partial, j0, lo_t, hi_t, c, st_cur + R::TILE,
                                                p.cap_in2, p.cap_out);
            else step_mfma<D, BN, BF16, true, true>(st, q, st_prev + R::TILE, st_cur);
            const int j3 = tile_key(jt + kStages - 1);
            const bool load3 = lead && jt + kStages - 1 < n;
            int page = 0;
            if (load3) page = win[R::slot(j3, first, p.bs_log2, w)];
            // tile jt+1 must have landed; tile jt+2, issued after it, may stay in
            // flight
            if (lead && jt + 1 < n) {
                if (jt + 2 < n) __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::LOADS_PER_TILE));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            block_barrier();
            // phase 2 (after the last tile the lead's QK reads a stale stage;
            // those scores are never used)
            if (lead) {
                const uint32_t st3 = ring_lds + ((jt + kStages - 1) % kStages) * R::STAGE;
                const bool spread = load3 && R::whole(j3, kv_len, w);
                if (load3 && !spread)
                    ld.issue(st3, p.k_cache, p.v_cache, win, first, j3, kv_len, p.bs_log2,
                             tok_stride, head_off, w, page);
                typename R::Src sr{p.k_cache, p.v_cache};
                if (spread)
                    sr = R::src(p.k_cache, p.v_cache, page, j3, w, p.bs_log2, tok_stride, head_off);
                step_mfma<D, BN, BF16, true, true>(st, q, st_cur + R::TILE, st_next,
                                                   Hook{ld, sr, st3, w, spread});
            } else {
                phase_softmax<D, BN, BF16, CAP>(st, partial, j0, lo_t, hi_t, c, st_cur + R::TILE,
                                                p.cap_in2, p.cap_out);
            }
            block_barrier();
        }
        if (!lead && n > 0) {
            step_mfma<D, BN, BF16, true, false>(st, q, ring + ((n - 1) % kStages) * R::STAGE + R::TILE,
                                                ring);
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) st.pb[kb][0] = st.pb[kb][1] = u32x4_t{0u, 0u, 0u, 0u};
        }
        block_barrier();   // the next chunk's window and ring refill start after all reads
    }

    const float l = st.lpart + xor32(st.lpart);
    if (valid) {
        const int64_t rowi = (int64_t)(q_start + tok) * p.num_heads + head;
        store_row<D, BF16>(st.o, l, p.out + rowi * D);
        if (p.lse != nullptr && g == 0)
            p.lse[rowi] = l > 0.f ? (st.m + __builtin_log2f(l)) * kLn2 : kNegInf;
    }
}

namespace {

template <int D, int BN, int QB, int NW, bool BF16, bool CAP, bool BSP>
hipError_t launch_cfg(const PrefillParams& p0, int max_seqlen_q, hipStream_t s) {
    constexpr int BM = NW * QB * 32;
    PrefillParams p = p0;
    const int tokens_per_tile = BM >> p.pack_log2;
    p.n_qtiles = (max_seqlen_q + tokens_per_tile - 1) / tokens_per_tile;
    const int64_t grid = 8 * tiles_per_xcd(p.batch, p.n_head_groups, p.total_q, max_seqlen_q,
                                           tokens_per_tile);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_paged_prefill<D, BN, QB, NW, BF16, CAP, BSP>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace

// Tile configurations (BN keys per tile, QB query blocks of 32 rows per wave,
// NW waves per workgroup).
#ifndef ATTN_PREFILL_D128
#define ATTN_PREFILL_D128 64, 1, 8
#endif
#ifndef ATTN_PREFILL_D64
#define ATTN_PREFILL_D64 64, 1, 8
#endif

namespace {

template <int D, int BN, int QB, int NW, bool BF16, bool BSP>
hipError_t launch_sparse(const PrefillParams& p, int max_seqlen_q, hipStream_t s) {
    return p.cap_out > 0.f ? launch_cfg<D, BN, QB, NW, BF16, true, BSP>(p, max_seqlen_q, s)
                           : launch_cfg<D, BN, QB, NW, BF16, false, BSP>(p, max_seqlen_q, s);
}

template <int D, int BN, int QB, int NW, bool BF16>
hipError_t launch_cap(const PrefillParams& p, int max_seqlen_q, hipStream_t s) {
    if (p.bm_kv_num != nullptr) {
        static_assert(BN == 64, "block-sparse key blocks are multiples of 64 keys");
        return launch_sparse<D, BN, QB, NW, BF16, true>(p, max_seqlen_q, s);
    }
    return launch_sparse<D, BN, QB, NW, BF16, false>(p, max_seqlen_q, s);
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillParams& p, int head_size, bool bf16,
                                int max_seqlen_q, hipStream_t s) {
    if (head_size == 128) {
        return bf16 ? launch_cap<128, ATTN_PREFILL_D128, true>(p, max_seqlen_q, s)
                    : launch_cap<128, ATTN_PREFILL_D128, false>(p, max_seqlen_q, s);
    }
    if (head_size == 64) {
        return bf16 ? launch_cap<64, ATTN_PREFILL_D64, true>(p, max_seqlen_q, s)
                    : launch_cap<64, ATTN_PREFILL_D64, false>(p, max_seqlen_q, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
