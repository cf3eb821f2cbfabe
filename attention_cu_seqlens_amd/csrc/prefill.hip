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
// Work decomposition needs no device->host sync: the host sizes the grid from
// max_seqlen_q; workgroup ids map to (query tile, sequence, head group) with
// the LAST query tiles first (the longest causal rows start earliest), and a
// workgroup whose tile lies past its sequence's end exits.
//
// Masks reduce to one visible key interval [lo, hi) per query row: causal
// (bottom-right) and patch bound hi, document ids (non-decreasing within a
// sequence) bound both.  Each wave classifies every key tile as empty (skip),
// full (no per-element test) or partial from the extreme intervals of its
// rows.

#include "device_common.h"
#include "kernels.h"

namespace attn {

namespace {

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ int upper_bound_i32(const int32_t* a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

}  // namespace

template <int D, int BN, int QB, int NW, bool BF16>
__global__ __launch_bounds__(NW * 64) void k_paged_prefill(PrefillParams p) {
    constexpr int NT = NW * 64;
    constexpr int BM = NW * QB * 32;
    using Tile = PagedTile16<D, BN, NT, false>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Tile::BYTES];
    __shared__ int wave_range[2][NW];
    __shared__ int win[PAGE_WIN + 1];

    int u = blockIdx.x;
    const int hg = u % p.n_head_groups;
    u /= p.n_head_groups;
    const int b = u % p.batch;
    const int qt = p.n_qtiles - 1 - u / p.batch;

    const int q_start = p.cu_q[b];
    const int q_len = p.cu_q[b + 1] - q_start;
    const int tok0 = qt * (BM >> p.pack_log2);
    if (tok0 >= q_len) return;
    const int kv_start = p.cu_kv[b];
    const int kv_len = p.cu_kv[b + 1] - kv_start;
    const int h0 = hg << p.pack_log2;
    const int hk = h0 / p.group;
    const bool neg = p.c < 0.f;
    const float c = fabsf(p.c);

    const int tid = threadIdx.x;
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 31, g = lane >> 5;

    RowsState<D, QB> st;
    st.init();
    int tok[QB], head[QB];
    bool valid[QB];
    int my_lo = 0x7fffffff, my_hi = -0x7fffffff, my_lo_max = -0x7fffffff, my_hi_min = 0x7fffffff;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int r = (w * QB + qb) * 32 + col;
        tok[qb] = tok0 + (r >> p.pack_log2);
        head[qb] = h0 + (r & ((1 << p.pack_log2) - 1));
        valid[qb] = tok[qb] < q_len;
        const uint16_t* qp =
            p.q + ((int64_t)(q_start + tok[qb]) * p.num_heads + head[qb]) * D + 8 * g;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (valid[qb]) v = *reinterpret_cast<const u32x4_t*>(qp + 16 * t);
            st.q[qb][t] = neg ? neg16x8(v) : v;
        }
        int lo = 0, hi = kv_len;
        if (valid[qb]) {
            if (p.mask & kMaskCausal) hi = min(hi, tok[qb] + (kv_len - q_len) + 1);
            if (p.mask & kMaskPatch) hi = min(hi, p.q_ids[q_start + tok[qb]] + 1);
            if (p.mask & kMaskDocument) {
                const int doc = p.q_ids[q_start + tok[qb]];
                lo = lower_bound_i32(p.kv_ids + kv_start, kv_len, doc);
                hi = min(hi, upper_bound_i32(p.kv_ids + kv_start, kv_len, doc));
            }
            if (hi < lo) hi = lo;
            my_lo = min(my_lo, lo);
            my_hi = max(my_hi, hi);
            my_lo_max = max(my_lo_max, lo);
            my_hi_min = min(my_hi_min, hi);
        } else {
            lo = 0;
            hi = 0;
        }
        st.lo[qb] = lo;
        st.hi[qb] = hi;
    }
    // Wave extremes over valid rows; an all-invalid wave gets an empty range.
    const int w_lo = wave_min(my_lo), w_hi = wave_max(my_hi);
    const int w_lo_max = wave_max(my_lo_max), w_hi_min = wave_min(my_hi_min);
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
    kv_begin &= ~15;   // 16-key aligned: a V unit never straddles a page

    const int32_t* table = p.block_table + (int64_t)b * p.mbps;
    const int n_blocks = (kv_len + (1 << p.bs_log2) - 1) >> p.bs_log2;
    const int tok_stride = p.num_kv_heads * D;
    const int head_off = hk * D;
    const int chunk_keys = PAGE_WIN << p.bs_log2;   // a multiple of BN
    Tile ld;

    // Key chunks of PAGE_WIN blocks: stage the chunk's block ids, then stream
    // its tiles with the next tile's loads in flight during the current one.
    for (int cs = kv_begin; cs < kv_end; cs += chunk_keys) {
        const int n_tiles = (min(kv_end, cs + chunk_keys) - cs + BN - 1) / BN;
        const int first = cs >> p.bs_log2;
        fill_page_window(win, table, first, n_blocks, tid, NT);
        __syncthreads();
        ld.load(p.k_cache, p.v_cache, win, first, cs, kv_len, p.bs_log2, tok_stride, head_off,
                tid);
        ld.store(smem, cs, kv_len, tid);
        __syncthreads();
        for (int it = 0; it < n_tiles; ++it) {
            const int j = cs + it * BN;
            const uint8_t* cur = smem + (it & 1) * Tile::BYTES;
            const bool has_next = it + 1 < n_tiles;
            if (has_next)
                ld.load(p.k_cache, p.v_cache, win, first, j + BN, kv_len, p.bs_log2, tok_stride,
                        head_off, tid);
            if (w_any && j < w_hi && j + BN > w_lo) {
                if (j >= w_lo_max && j + BN <= w_hi_min)
                    tile_step<D, BN, BN / 32, QB, BF16, false>(st, cur, j, 0, c);
                else
                    tile_step<D, BN, BN / 32, QB, BF16, true>(st, cur, j, 0, c);
            }
            if (has_next) ld.store(smem + ((it + 1) & 1) * Tile::BYTES, j + BN, kv_len, tid);
            __syncthreads();
        }
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        if (!valid[qb]) continue;
        const int64_t row = (int64_t)(q_start + tok[qb]) * p.num_heads + head[qb];
        f32x16_t o_db[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o_db[db] = st.o[db][qb];
        store_row<D, BF16>(o_db, st.l[qb], p.out + row * D);
        if (p.lse != nullptr && g == 0)
            p.lse[row] = st.l[qb] > 0.f ? (st.m[qb] + __builtin_log2f(st.l[qb])) * kLn2 : kNegInf;
    }
}

namespace {

template <int D, int BN, int QB, int NW, bool BF16>
hipError_t launch_cfg(const PrefillParams& p0, int max_seqlen_q, hipStream_t s) {
    constexpr int BM = NW * QB * 32;
    PrefillParams p = p0;
    const int tokens_per_tile = BM >> p.pack_log2;
    p.n_qtiles = (max_seqlen_q + tokens_per_tile - 1) / tokens_per_tile;
    const int64_t grid = (int64_t)p.n_qtiles * p.batch * p.n_head_groups;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_paged_prefill<D, BN, QB, NW, BF16>), dim3((unsigned)grid),
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
#define ATTN_PREFILL_D64 128, 1, 8
#endif

hipError_t launch_paged_prefill(const PrefillParams& p, int head_size, bool bf16,
                                int max_seqlen_q, hipStream_t s) {
    if (head_size == 128) {
        return bf16 ? launch_cfg<128, ATTN_PREFILL_D128, true>(p, max_seqlen_q, s)
                    : launch_cfg<128, ATTN_PREFILL_D128, false>(p, max_seqlen_q, s);
    }
    if (head_size == 64) {
        return bf16 ? launch_cfg<64, ATTN_PREFILL_D64, true>(p, max_seqlen_q, s)
                    : launch_cfg<64, ATTN_PREFILL_D64, false>(p, max_seqlen_q, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
