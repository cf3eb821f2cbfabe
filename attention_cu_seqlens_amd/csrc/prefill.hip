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
// the last tile exit at once.  Head size 128 runs the eight-wave kernel
// below, one workgroup per CU.  Head size 64 runs four-wave workgroups,
// several per CU (k_paged_prefill_pair), except under stored block lists,
// where it keeps the eight-wave kernel; there, when every sequence has the
// same length (total_q = batch * max_seqlen_q), one workgroup per CU walks a
// fixed snake of its XCD's tiles (no dispatch between tiles; at head size
// 128 that loop made the compiler spill).
//
// Masks reduce to one visible key interval [lo, hi) per query row: causal
// (bottom-right) and patch bound hi, document ids (non-decreasing within a
// sequence) bound both.  Each wave classifies every key tile as empty (skip),
// full (no per-element test) or partial from the extreme intervals of its
// rows.

#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "kernels.h"
#include "ring.h"

namespace attn {

// Ring depth: up to kStages - 1 tiles in flight while one is consumed.
constexpr int kStages = 4;

// Per-wave pipeline state of one 32-row block.
template <int D, int BN>
struct PrefillWave {
    f32x16_t s[BN / 32];      // scores of the tile waiting for its softmax
    u32x4_t pb[BN / 32][2];   // probabilities of the tile waiting for its P.V
    f32x16_t o[D / 32];
    float m, lpart, alpha;
    bool need;
};

// Softmax phase (VALU): mask the scores of the tile at key j0 when partial,
// then probabilities into pb (scores capped first with CAP).
template <int D, int BN, bool BF16, bool CAP>
__device__ __forceinline__ void phase_softmax(PrefillWave<D, BN>& st, bool partial, int j0, int lo,
                                              int hi, float c, float cap_in2, float cap_out) {
    if (partial) {
        // key k of register r is visible iff lo <= k < hi, i.e. the unsigned
        // k - lo is below hi - lo (hi >= lo): one add, one compare and one
        // select per score
        const uint32_t off = (uint32_t)(j0 + 4 * (lane_id() >> 5) - lo);
        const uint32_t width = (uint32_t)(hi - lo);
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t k = off + (uint32_t)(kb * 32 + 8 * (r >> 2) + (r & 3));
                if (!(k < width)) st.s[kb][r] = kNegInf;
            }
    }
    softmax_tile<BN, BF16, CAP>(st.s, c, st.m, st.lpart, st.pb, st.alpha, st.need, cap_in2,
                                cap_out);
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
    mfma_stream16<D, BN, BF16, PV, QK>(st.o, st.s, st.pb, q, v_tile, k_tile, hook);
    __builtin_amdgcn_s_setprio(0);
}

template <int D, int BN, int QB, int NW, bool BF16, bool CAP, bool BSP, bool PERSIST>
__global__ __launch_bounds__(NW * 64) void k_paged_prefill(PrefillParams p) {
    static_assert(QB == 1 && NW == 8, "two groups of four single-block waves");
    constexpr int BM = NW * 32;
    static_assert(BM == kPrefillRows, "rows per workgroup as the host assumes");
    static_assert(PAGE_WIN * 64 / BN <= NW * 64, "a chunk's tiles fit one per thread");
    using R = Ring16<D, BN, NW / 2>;
    // Head size 64: the lead waves issue the K rows of tile jt + 3 after their
    // MFMA phase, the trailing waves only the V rows of tile jt + 2 (byte ->
    // patch cross attention 0.122 against 0.130 ms).  At 128 the lead waves'
    // loads lengthen the varlen prefill (0.887 against 0.833 ms).
    constexpr bool kLeadK = D == 64;
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

    // Kernel arguments the set-up reads, fetched together up front (left to
    // itself the compiler reloads each one where it is used, one dependent
    // scalar round trip after another).
    int a_group = p.group, a_heads = p.num_heads, a_window = p.window;
    uint32_t a_mask = p.mask;
    float a_c = p.c;
    const uint16_t* a_q = p.q;
    asm volatile("" : "+s"(a_group), "+s"(a_heads), "+s"(a_window), "+s"(a_mask), "+s"(a_c),
                 "+s"(a_q));
    // Persistent form: workgroup g of an XCD takes items g, then 2G-1-g,
    // then 2G+g, ... of the XCD's list (G workgroups per XCD; a snake, so
    // the longest-first order of each unit's tiles pairs long with short).
    const int g_wg = blockIdx.x >> 3;
    for (int j = 0;; ++j) {
        int k_item = g_wg;
        if constexpr (PERSIST) {
            k_item = j * p.wg_per_xcd + ((j & 1) ? p.wg_per_xcd - 1 - g_wg : g_wg);
        } else {
            if (j > 0) break;
        }
        int b, hg, qt;
        SeqSpan sp;
        if (!map_tile(p.cu_q, p.cu_kv, p.batch, p.n_head_groups, BM >> p.pack_log2, blockIdx.x & 7,
                      k_item, b, hg, qt, sp))
            break;

        const int q_start = sp.q_start;
        const int q_len = sp.q_len;
        const int tok0 = qt * (BM >> p.pack_log2);
        const int kv_start = sp.kv_start;
        const int kv_len = sp.kv_len;
        const int h0 = hg << p.pack_log2;
        const int hk = h0 / a_group;
        const bool neg = a_c < 0.f;
        const int32_t* table = p.block_table + (int64_t)b * p.mbps;
        const int n_blocks = (kv_len + (1 << p.bs_log2) - 1) >> p.bs_log2;
        // Without a document mask, a local window or block lists every row's
        // visible keys start at key 0, so the first key chunk starts there: its
        // block ids are requested now, and their round trip overlaps the row
        // intervals and the set-up barrier instead of following them.
        const bool win_early = !BSP && !(a_mask & kMaskDocument) && a_window <= 0;
        if (win_early) fill_page_window(win, table, 0, n_blocks, threadIdx.x, NW * 64);
        // |scale| log2(e), at least 1e-30: a masked score (-inf) then always
        // gives exp2(-inf) = 0, and a zero scale still gives every visible key
        // weight exactly 1 (scores times 1e-30 are far below half an ulp of 1)
        const float c = fmaxf(fabsf(a_c), 1e-30f);

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
        // while the other computes a softmax.  The second group alone loads the
        // K/V ring, at the start of its softmax phase.
        const bool lead = w < NW / 2;

        // this lane's query row
        const int r = w * 32 + col;
        const int tok = tok0 + (r >> p.pack_log2);
        const int head = h0 + (r & ((1 << p.pack_log2) - 1));
        const bool valid = tok < q_len;
        int lo = 0, hi = 0;
        if (valid) {
            hi = kv_len;
            if (a_mask & kMaskCausal) hi = min(hi, tok + (kv_len - q_len) + 1);
            if (a_mask & kMaskPatch) hi = min(hi, p.q_ids[q_start + tok] + 1);
            if (a_mask & kMaskDocument) {
                const int doc = p.q_ids[q_start + tok];
                lo = lower_bound_i32(p.kv_ids + kv_start, kv_len, doc);
                hi = min(hi, upper_bound_i32(p.kv_ids + kv_start, kv_len, doc));
            }
            // local window: keys after the query's own position minus the window
            if (a_window > 0) lo = max(lo, tok + (kv_len - q_len) - a_window + 1);
            if (hi < lo) hi = lo;
        }
        // Q into this wave's slice of the ring (stages 0 and 1, free until the
        // first key chunk's loads), laid out like a K tile: row rr (the wave's
        // rows in order) holds 16-byte chunk c at c ^ swz(rr).  One direct load
        // moves 64 / (D / 8) whole rows -- with GQA packing, consecutive heads of
        // one token, contiguous in memory -- where loading the operand layout
        // straight into registers touched 32 rows per instruction.  A row past
        // the sequence end reads row tok0 instead (its keys are all masked and it
        // is never stored).  Issued after the row intervals: a mask whose interval
        // needs loads (patch, document) waits for them, and such a wait would
        // also wait for any load issued before.
        static_assert(NW * 32 * 2 * D <= 2 * R::STAGE, "Q slices fit stages 0 and 1");
        uint8_t* const q_slice = ring + w * 32 * 2 * D;
        {
            constexpr int CPR = D / 8, RPI = 64 / CPR;
            const int ch = lane % CPR;
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
                const int rr = i * RPI + lane / CPR;
                const int rw = w * 32 + rr;
                const int tk = tok0 + (rw >> p.pack_log2);
                const int hd = h0 + (rw & ((1 << p.pack_log2) - 1));
                const uint16_t* src = a_q + ((int64_t)(q_start + (tk < q_len ? tk : tok0)) * a_heads + hd) * D +
                                      8 * (ch ^ swz<D>(rr));
                dma16(src, lds_addr(q_slice + i * 1024));
            }
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

        // Q operand from the wave's slice (its direct loads have landed after
        // the wait; each wave reads only its own slice): lane (col, g) takes
        // chunks 2t + g of row col.  Every wave's reads complete before the
        // barrier that precedes the first ring load into these stages.
        u32x4_t q[D / 16];
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        {
            const uint32_t lq = (uint32_t)(col * 2 * D + ((g ^ swz<D>(col)) << 4));
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                q[t] = *reinterpret_cast<const u32x4_t*>(q_slice + (lq ^ (uint32_t)(t << 5)));
                if (neg) q[t] = neg16x8(q[t]);
            }
        }

        const int tok_stride = p.num_kv_heads * D;
        const int head_off = hk * D;
        const int chunk_keys = PAGE_WIN << p.bs_log2;   // a multiple of BN
        R ld;
        const int wl = w & (NW / 2 - 1);   // this wave's index within its group
        ld.init(lane, wl, tok_stride);
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
        //   lead:  softmax(j), then P.V(j) and QK(j+1)
        //   trail: P.V(j-1) and QK(j), then the ring loads, then softmax(j)
        // with one workgroup barrier per tile.  A tile then takes the longer of
        // the two waves' totals rather than the sum of the longer side of each
        // half (two barriers per tile measured 4% slower on the varlen workload,
        // 8% on byte->patch cross attention).  The trailing waves alone load the
        // ring, V rows of tile j+2 and K rows of tile j+3: the lead waves' MFMA
        // stream is bound by its LDS operand reads, and loads issued from it
        // (which write LDS too) cost it about 70 cycles each, against about 40
        // from the trailing side.
        // The trailing waves' first P.V of a chunk multiplies P = 0 (pb zeroed
        // here and after each chunk) by the V tile of the last stage: zeroed here
        // (uninitialised LDS could hold NaN codes), later a finite cache tile.
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) st.pb[kb][0] = st.pb[kb][1] = u32x4_t{0u, 0u, 0u, 0u};
        for (int i = tid; i < R::TILE / 16; i += NW * 64)
            *reinterpret_cast<u32x4_t*>(ring + (kStages - 1) * R::STAGE + R::TILE + 16 * i) =
                u32x4_t{0u, 0u, 0u, 0u};
        for (int cs = kv_begin; cs < kv_end; cs += chunk_keys) {
            int n = (min(kv_end, cs + chunk_keys) - cs + BN - 1) / BN;
            const int first = cs >> p.bs_log2;
            if (!(win_early && cs == 0)) fill_page_window(win, table, first, n_blocks, tid, NW * 64);
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
            // Tile jt, between barriers:
            //   lead:  softmax(jt); P.V(jt), QK(jt+1) [; K rows of tile jt+3]
            //   trail: P.V(jt-1), QK(jt); V rows of tile jt+2 [, K rows of tile
            //          jt+3]; softmax(jt)
            // (the K rows of tile jt+3 from the lead waves at head size 64, from
            // the trailing waves at 128).  V(jt+2) goes into the stage of tile
            // jt-2, whose V was last read by P.V(jt-2) in tile jt-1; K(jt+3) into
            // the stage of tile jt-1, whose K was last read by QK(jt-1) in tile
            // jt-1.  Before the barrier each wave waits for its own loads among
            // V(jt+1) and K(jt+2), which the next tile reads (P.V; the lead's
            // QK(jt+2)).
            {
                // trailing waves: K(0), V(0), K(1), V(1), K(2); then K(0), V(0),
                // K(1) must have landed (the lead's QK(0), softmax(0), QK(1))
                if (!lead) {
#pragma unroll
                    for (int k = 0; k < kStages - 1; ++k)
                        if (k < n) {
                            const int jk = tile_key(k);
                            const int pg = win[R::slot(jk, first, p.bs_log2, wl)];
                            ld.issue_half(false, ring_lds + k * R::STAGE, p.k_cache, p.v_cache, win,
                                          first, jk, kv_len, p.bs_log2, tok_stride, head_off, wl, pg);
                            if (k < kStages - 2)
                                ld.issue_half(true, ring_lds + k * R::STAGE, p.k_cache, p.v_cache,
                                              win, first, jk, kv_len, p.bs_log2, tok_stride,
                                              head_off, wl, pg);
                        }
                    static_assert(kStages == 4, "wait counts below");
                    if (n > 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * R::IPW));
                    else if (n > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::IPW));
                    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                }
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
                if (lead) {
                    phase_softmax<D, BN, BF16, CAP>(st, partial, j0, lo_t, hi_t, c, p.cap_in2,
                                                    p.cap_out);
                    step_mfma<D, BN, BF16, true, true>(st, q, st_cur + R::TILE, st_next);
                    if constexpr (kLeadK) {
                        if (jt + 3 < n) {
                            const int j3 = tile_key(jt + 3);
                            ld.issue_half(false, ring_lds + ((jt + 3) % kStages) * R::STAGE,
                                          p.k_cache, p.v_cache, win, first, j3, kv_len, p.bs_log2,
                                          tok_stride, head_off, wl,
                                          win[R::slot(j3, first, p.bs_log2, wl)]);
                        }
                        // this wave's K(jt+2) landed: only K(jt+3) may stay
                        if (jt + 3 < n) __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::IPW));
                        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    }
                } else {
                    step_mfma<D, BN, BF16, true, true>(st, q, st_prev + R::TILE, st_cur);
                    // issue order V(jt+2), K(jt+3): waiting for V(jt+1) and K(jt+2)
                    // leaves only the loads of this tile in flight
                    if (jt + 2 < n) {
                        const int j2 = tile_key(jt + 2);
                        ld.issue_half(true, ring_lds + ((jt + 2) % kStages) * R::STAGE, p.k_cache,
                                      p.v_cache, win, first, j2, kv_len, p.bs_log2, tok_stride,
                                      head_off, wl, win[R::slot(j2, first, p.bs_log2, wl)]);
                    }
                    if (!kLeadK && jt + 3 < n) {
                        const int j3 = tile_key(jt + 3);
                        ld.issue_half(false, ring_lds + ((jt + 3) % kStages) * R::STAGE, p.k_cache,
                                      p.v_cache, win, first, j3, kv_len, p.bs_log2, tok_stride,
                                      head_off, wl, win[R::slot(j3, first, p.bs_log2, wl)]);
                    }
                    phase_softmax<D, BN, BF16, CAP>(st, partial, j0, lo_t, hi_t, c, p.cap_in2,
                                                    p.cap_out);
                    // the probabilities are computed before the wait below (left to
                    // itself the compiler sinks the exponentials after it)
                    asm volatile("" ::"v"(st.pb[0][0]), "v"(st.pb[0][1]), "v"(st.pb[BN / 32 - 1][0]),
                                 "v"(st.pb[BN / 32 - 1][1]), "v"(st.lpart));
                    // this wave's V(jt+1) and K(jt+2) landed: only V(jt+2), K(jt+3) may stay
                    {
                        const int inflight =
                            (jt + 2 < n ? R::IPW : 0) + (!kLeadK && jt + 3 < n ? R::IPW : 0);
                        if (inflight == 2 * R::IPW) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * R::IPW));
                        else if (inflight == R::IPW) __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::IPW));
                        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    }
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

        const float l = pair_sum(st.lpart);
        // With no key tile the output slices below could overlap another wave's
        // Q slice still being read: wait for every wave first.
        if (kv_begin >= kv_end) block_barrier();
        // O goes out through this wave's slice of the ring: every wave has passed
        // the last chunk's closing barrier (nothing reads the ring any more), and
        // the slices lie below the last stage's V half, which was zeroed before
        // the key loop without a barrier after it.
        static_assert(NW * kStoreSliceBytes<D> <= (kStages - 1) * R::STAGE + R::TILE,
                      "output slices clear of the zeroed V half");
        store_rows_lds<D, BF16>(st.o, l, ring + w * kStoreSliceBytes<D>, [&](int rr) -> uint16_t* {
            const int rw = w * 32 + rr;
            const int tk = tok0 + (rw >> p.pack_log2);
            const int hd = h0 + (rw & ((1 << p.pack_log2) - 1));
            return tk < q_len ? p.out + ((int64_t)(q_start + tk) * p.num_heads + hd) * D : nullptr;
        });
        if (valid && p.lse != nullptr && g == 0) {
            const int64_t rowi = (int64_t)(q_start + tok) * p.num_heads + head;
            p.lse[rowi] = l > 0.f ? (st.m + __builtin_log2f(l)) * kLn2 : kNegInf;
        }
        // the next item's loads overwrite LDS this item's waves may still read
        if constexpr (PERSIST) __syncthreads();
    }
}


// Head size 64, dense or masked (no stored block lists): several small
// workgroups per CU instead of one.  A workgroup is four waves (one per
// SIMD) holding 128 packed query rows, and its K/V ring has two stages
// (35 KB of LDS; built for four waves per SIMD, 128 registers), so four fit
// on a CU and each SIMD runs one wave of each (three at the 136 registers
// the compiler picks unbounded: 1.1% slower on byte -> patch cross
// attention).  The workgroups are not in step: while one is in its set-up,
// epilogue or a barrier, the others' MFMA and softmax work keeps the SIMD
// busy.  Byte -> patch cross attention's workgroups see short key ranges, so
// set-up and epilogue are a large share of each, which the eight-wave
// kernel (one workgroup per CU) cannot overlap.  At head size 128 (66 KB,
// 193 registers: two per CU) the form measured even with the eight-wave
// kernel, which stays there.
// Per key tile each wave waits for its own loads of the tile, meets the
// others at the barrier (after which the other stage is free: its last
// reads were the previous tile's), runs QK on the current stage, issues its
// 16 key rows of the next tile into the other stage, then runs the softmax
// and P.V.  (Measured in the head-size-128 form against the eight-wave
// kernel: loads issued ahead of QK 2.6% slower, between QK and the softmax
// 0.8-2% faster, between the softmax and P.V even.)
template <int D, bool BF16, bool CAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_paged_prefill_pair(
    PrefillParams p) {
    constexpr int NW = 4, BN = 64, BM = NW * 32;
    using R = Ring16<D, BN, NW>;
    static_assert(NW * 32 * 2 * D <= R::STAGE, "Q slices fit stage 0");
    static_assert(NW * kStoreSliceBytes<D> <= 2 * R::STAGE, "output slices fit the ring");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * R::STAGE];
    __shared__ int wave_range[2][NW];
    __shared__ int win[PAGE_WIN + 1];

    int a_group = p.group, a_heads = p.num_heads, a_window = p.window;
    uint32_t a_mask = p.mask;
    float a_c = p.c;
    const uint16_t* a_q = p.q;
    asm volatile("" : "+s"(a_group), "+s"(a_heads), "+s"(a_window), "+s"(a_mask), "+s"(a_c),
                 "+s"(a_q));
    int b, hg, qt;
    SeqSpan sp;
    if (!map_tile(p.cu_q, p.cu_kv, p.batch, p.n_head_groups, BM >> p.pack_log2, blockIdx.x & 7,
                  blockIdx.x >> 3, b, hg, qt, sp))
        return;
    const int q_start = sp.q_start, q_len = sp.q_len;
    const int tok0 = qt * (BM >> p.pack_log2);
    const int kv_start = sp.kv_start, kv_len = sp.kv_len;
    const int h0 = hg << p.pack_log2;
    const int hk = h0 / a_group;
    const bool neg = a_c < 0.f;
    const int32_t* table = p.block_table + (int64_t)b * p.mbps;
    const int n_blocks = (kv_len + (1 << p.bs_log2) - 1) >> p.bs_log2;
    const bool win_early = !(a_mask & kMaskDocument) && a_window <= 0;
    if (win_early) fill_page_window(win, table, 0, n_blocks, threadIdx.x, NW * 64);
    const float c = fmaxf(fabsf(a_c), 1e-30f);

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int w = wave_id();
    const int col = lane & 31, g = lane >> 5;
    const int r = w * 32 + col;
    const int tok = tok0 + (r >> p.pack_log2);
    const int head = h0 + (r & ((1 << p.pack_log2) - 1));
    const bool valid = tok < q_len;
    int lo = 0, hi = 0;
    if (valid) {
        hi = kv_len;
        if (a_mask & kMaskCausal) hi = min(hi, tok + (kv_len - q_len) + 1);
        if (a_mask & kMaskPatch) hi = min(hi, p.q_ids[q_start + tok] + 1);
        if (a_mask & kMaskDocument) {
            const int doc = p.q_ids[q_start + tok];
            lo = lower_bound_i32(p.kv_ids + kv_start, kv_len, doc);
            hi = min(hi, upper_bound_i32(p.kv_ids + kv_start, kv_len, doc));
        }
        if (a_window > 0) lo = max(lo, tok + (kv_len - q_len) - a_window + 1);
        if (hi < lo) hi = lo;
    }
    // Q of this wave's rows into its slice of stage 0 by direct loads of whole
    // rows (a row past the sequence end reads row tok0; never stored)
    uint8_t* const q_slice = ring + w * 32 * 2 * D;
    {
        constexpr int CPR = D / 8, RPI = 64 / CPR;
        const int ch = lane % CPR;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int rr = i * RPI + lane / CPR;
            const int rw = w * 32 + rr;
            const int tk = tok0 + (rw >> p.pack_log2);
            const int hd = h0 + (rw & ((1 << p.pack_log2) - 1));
            const uint16_t* src = a_q + ((int64_t)(q_start + (tk < q_len ? tk : tok0)) * a_heads + hd) * D +
                                  8 * (ch ^ swz<D>(rr));
            dma16(src, lds_addr(q_slice + i * 1024));
        }
    }
    const int w_lo = wave_min(valid ? lo : 0x7fffffff);
    const int w_hi = wave_max(valid ? hi : -0x7fffffff);
    const int w_lo_max = wave_max(valid ? lo : -0x7fffffff);
    const int w_hi_min = wave_min(valid ? hi : 0x7fffffff);
    const bool w_any = w_hi > w_lo;
    if (lane == 0) {
        wave_range[0][w] = w_any ? w_lo : 0x7fffffff;
        wave_range[1][w] = w_any ? w_hi : -0x7fffffff;
    }
    __syncthreads();
    int kv_begin = 0x7fffffff, kv_end = -0x7fffffff;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        kv_begin = min(kv_begin, wave_range[0][i]);
        kv_end = max(kv_end, wave_range[1][i]);
    }
    kv_begin = __builtin_amdgcn_readfirstlane(kv_begin & ~15);
    kv_end = __builtin_amdgcn_readfirstlane(kv_end);

    // Q operand from the wave's own slice; every wave's reads complete before
    // the first key chunk's barrier, after which the ring loads refill stage 0
    u32x4_t q[D / 16];
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    {
        const uint32_t lq = (uint32_t)(col * 2 * D + ((g ^ swz<D>(col)) << 4));
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            q[t] = *reinterpret_cast<const u32x4_t*>(q_slice + (lq ^ (uint32_t)(t << 5)));
            if (neg) q[t] = neg16x8(q[t]);
        }
    }

    const int tok_stride = p.num_kv_heads * D;
    const int head_off = hk * D;
    const int chunk_keys = PAGE_WIN << p.bs_log2;   // a multiple of BN
    R ld;
    ld.init(lane, w, tok_stride);
    const uint32_t ring_lds = lds_addr(ring);

    PrefillWave<D, BN> st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.o[db] = f32x16_t{};
    st.m = kNegInf;
    st.lpart = 0.f;
    st.alpha = 1.f;
    st.need = false;

    for (int cs = kv_begin; cs < kv_end; cs += chunk_keys) {
        const int n = (min(kv_end, cs + chunk_keys) - cs + BN - 1) / BN;
        const int first = cs >> p.bs_log2;
        if (!(win_early && cs == 0)) fill_page_window(win, table, first, n_blocks, tid, NW * 64);
        // the window is in place and every wave is done with the ring (its Q
        // reads, or the previous chunk's last tile): its LDS operations have
        // completed before it reaches the barrier
        __builtin_amdgcn_s_waitcnt(0xC07Fu);   // lgkmcnt(0)
        __syncthreads();
        auto issue = [&](int k) {
            const int jk = cs + k * BN;
            const int pg = win[R::slot(jk, first, p.bs_log2, w)];
            const uint32_t stage = ring_lds + (k & 1) * R::STAGE;
            ld.issue_half(false, stage, p.k_cache, p.v_cache, win, first, jk, kv_len, p.bs_log2,
                          tok_stride, head_off, w, pg);
            ld.issue_half(true, stage, p.k_cache, p.v_cache, win, first, jk, kv_len, p.bs_log2,
                          tok_stride, head_off, w, pg);
        };
        issue(0);
        for (int jt = 0; jt < n; ++jt) {
            const int j0 = cs + jt * BN;
            // this wave's rows of tile jt have landed; after the barrier every
            // wave's have, and nobody reads the other stage any more
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            block_barrier();
            const uint8_t* cur = ring + (jt & 1) * R::STAGE;
            const bool partial = !(w_any && j0 >= w_lo_max && j0 + BN <= w_hi_min);
            step_mfma<D, BN, BF16, false, true>(st, q, cur, cur);
            if (jt + 1 < n) issue(jt + 1);
            phase_softmax<D, BN, BF16, CAP>(st, partial, j0, lo, hi, c, p.cap_in2, p.cap_out);
            step_mfma<D, BN, BF16, true, false>(st, q, cur + R::TILE, cur);
        }
        block_barrier();   // the last tile's reads are done before the ring is reused
    }

    const float l = pair_sum(st.lpart);
    // with no key tile the output slices could overlap another wave's Q slice
    // still being read
    if (kv_begin >= kv_end) block_barrier();
    store_rows_lds<D, BF16>(st.o, l, ring + w * kStoreSliceBytes<D>, [&](int rr) -> uint16_t* {
        const int rw = w * 32 + rr;
        const int tk = tok0 + (rw >> p.pack_log2);
        const int hd = h0 + (rw & ((1 << p.pack_log2) - 1));
        return tk < q_len ? p.out + ((int64_t)(q_start + tk) * p.num_heads + hd) * D : nullptr;
    });
    if (valid && p.lse != nullptr && g == 0) {
        const int64_t rowi = (int64_t)(q_start + tok) * p.num_heads + head;
        p.lse[rowi] = l > 0.f ? (st.m + __builtin_log2f(l)) * kLn2 : kNegInf;
    }
}

namespace {

// Compute units per XCD of the current device.
hipError_t cus_per_xcd(int* out) {
    int n = 0;
    const hipError_t e = cu_count(&n);
    if (e != hipSuccess) return e;
    *out = std::max(1, n / 8);
    return hipSuccess;
}

template <int D, int BN, int QB, int NW, bool BF16, bool CAP, bool BSP>
hipError_t launch_cfg(const PrefillParams& p0, int max_seqlen_q, hipStream_t s) {
    constexpr int BM = NW * QB * 32;
    PrefillParams p = p0;
    const int tokens_per_tile = BM >> p.pack_log2;
    p.n_qtiles = (max_seqlen_q + tokens_per_tile - 1) / tokens_per_tile;
    const int64_t per_xcd = tiles_per_xcd(p.batch, p.n_head_groups, p.total_q, max_seqlen_q,
                                          tokens_per_tile);
    if (per_xcd <= 0) return hipSuccess;
    if (8 * per_xcd > 0x7fffffff) return hipErrorInvalidConfiguration;
    // Block lists at head size 64 with equal-length sequences (every query
    // tile of a unit count is known, the tiles' key ranges vary only along
    // each unit): one workgroup per CU runs a fixed snake of the XCD's items,
    // with no dispatch between items.  Ragged batches keep one workgroup per
    // item (the dispatcher balances their unequal lengths).
    const bool uniform = (int64_t)p.total_q == (int64_t)p.batch * max_seqlen_q;
    if constexpr (D == 64 && BSP) {
        if (uniform) {
            int cu = 0;
            hipError_t e = cus_per_xcd(&cu);
            if (e != hipSuccess) return e;
            p.wg_per_xcd = (int)std::min<int64_t>(per_xcd, cu);
            hipLaunchKernelGGL((k_paged_prefill<D, BN, QB, NW, BF16, CAP, BSP, true>),
                               dim3((unsigned)(8 * p.wg_per_xcd)), dim3(NW * 64), 0, s, p);
            return hipGetLastError();
        }
    }
    if constexpr (D == 64 && !BSP) {
        // four-wave workgroups, 128 rows each, several per CU
        constexpr int BM2 = 128;
        const int tt2 = BM2 >> p.pack_log2;
        p.n_qtiles = (max_seqlen_q + tt2 - 1) / tt2;
        const int64_t per_xcd2 = tiles_per_xcd(p.batch, p.n_head_groups, p.total_q, max_seqlen_q, tt2);
        if (8 * per_xcd2 > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((k_paged_prefill_pair<D, BF16, CAP>), dim3((unsigned)(8 * per_xcd2)),
                           dim3(256), 0, s, p);
        return hipGetLastError();
    } else {
        hipLaunchKernelGGL((k_paged_prefill<D, BN, QB, NW, BF16, CAP, BSP, false>),
                           dim3((unsigned)(8 * per_xcd)), dim3(NW * 64), 0, s, p);
        return hipGetLastError();
    }
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
