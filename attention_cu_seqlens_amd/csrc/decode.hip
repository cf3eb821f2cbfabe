// Paged GQA decode (one query token per sequence) for 16-bit dtypes on gfx950.
//
// Split-KV with a balanced schedule.  A unit is (sequence b, group hg of HP
// adjacent kv heads), HP = 4, 2 or 1, the largest that divides Hkv: the
// cache stores a key's kv heads side by side, so the HP heads' rows of one
// key are HP * D contiguous elements, and the unit's loads of a key cover
// them at once instead of one head's D elements at a stride of Hkv * D (an
// fp8 cache with 8 kv heads streamed one head at a time reads 128-byte
// pieces 1 KiB apart and runs about 15% below the same bytes read as whole
// rows).  Every unit's visible keys form a run of 32-key tiles; the runs are
// laid end to end in (b, hg) order and workgroup w takes tiles
// [w*C, (w+1)*C) of that list, so every workgroup streams the same number of
// tiles (the last one fewer) whatever the mix of lengths.  By default the
// grid is two workgroups per CU, all resident at once: no tail of long
// splits running alone and no workgroup turnover.  A workgroup's share is
// cut at unit boundaries into segments; in each, NW / HP waves serve each
// head of the group, taking interleaved 32-key tiles of its keys, each wave
// with its own online-softmax state for the G = Hq/Hkv query heads of its
// kv head (the 32 query columns of the MFMA, G of them live); the waves of a
// head merge in LDS and write one partial (unnormalised O, running max m,
// sum l) per query head: HP * G rows per segment.  A second kernel merges
// each unit's segments with the same logsumexp rule; its LSE output is the
// "OUTPUT_LOGSUMEXP" quantity of the FlexAttention kernel options shown in
// the blt issue "Cross Attention does not work on CPU and older GPUs".
//
// Segment (unit u, workgroup w) writes partial slot u + w: along the list
// either the unit or the workgroup index grows from one segment to the next,
// so the slots are distinct, and a unit's segments hold consecutive slots.
// The workgroup that runs a unit's first tile records the unit's first slot
// and segment count for the merge.  No device->host sync: the tile counts
// come from cu_seqlens_kv on the device; the host sizes the grid and the
// workspace from max_seqlen_kv.

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace attn {

template <int D, int NW, bool BF16, bool KV8>
struct DecodeLayout {
    // one wave, 32 keys; the fp8 cache loader fills the same 16-bit tile
    using Tile = std::conditional_t<KV8, PagedTile8<D, BF16>, PagedTile16<D, 32, 64, true>>;
    static constexpr int WIN_OFF = NW * Tile::BYTES;
    static constexpr int TILE_BYTES = WIN_OFF + (PAGE_WIN + 1) * 4;
    static constexpr int RED_BYTES = NW * 32 * (D + 2) * 4;   // merge space, G <= 32
    static constexpr int LDS_BYTES = TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES;
};

// First key of the tiles a sequence of kv_len keys runs: 0, or with a local
// window of W keys the start of its last W keys rounded down to 32 (tiles
// stay 32-key aligned; the keys before the window are masked).
__device__ __forceinline__ int decode_klo(int kv_len, int window) {
    return (window > 0 ? max(0, kv_len - window) : 0) & ~31;
}
__device__ __forceinline__ int decode_tiles(int kv_len, int window) {
    return kv_len > 0 ? (kv_len - decode_klo(kv_len, window) + 31) >> 5 : 0;
}

template <int D, int NW, bool BF16, bool CAP, bool KV8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_paged_decode(DecodeParams p) {
    static_assert(NW % 4 == 0, "every head pack (1, 2, 4) divides the waves");
    using L = DecodeLayout<D, NW, BF16, KV8>;
    using Tile = typename L::Tile;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int* win = reinterpret_cast<int*>(smem + L::WIN_OFF);
    const int tid = threadIdx.x;
    const int lane = lane_id(), w = wave_id();
    const int Hkv = p.num_kv_heads;
    const int HP = p.head_pack;   // kv heads per unit: 1, 2 or 4, divides NW
    const int Hu = Hkv / HP;      // units per sequence
    const int WPH = NW / HP;      // waves per kv head
    const int hsub = w / WPH;     // this wave's head within the unit
    const int wt = w - hsub * WPH;
    const int wg = blockIdx.x;

    // The tile list: total length, this workgroup's share [start, end) and
    // the unit holding its first tile.  Wave-uniform, computed by every wave.
    int total = 0;
    for (int base = 0; base < p.batch; base += 64) {
        const int bb = base + lane;
        const int t = bb < p.batch ? decode_tiles(p.cu_kv[bb + 1] - p.cu_kv[bb], p.window) : 0;
        total += __builtin_amdgcn_readlane(wave_incl_scan(t), 63);
    }
    total *= Hu;
    const int C = p.split_tiles > 0
                      ? p.split_tiles
                      : max(kDecodeMinSegTiles, (total + (int)gridDim.x - 1) / (int)gridDim.x);
    if ((int64_t)wg * C >= total) return;
    const int start = wg * C;
    const int end = min(total, start + C);
    int b = 0, hg = 0, t0 = 0;
    {
        int acc = 0;   // tiles per unit of the sequences before `base`
        for (int base = 0; base < p.batch; base += 64) {
            const int bb = base + lane;
            const int t = bb < p.batch ? decode_tiles(p.cu_kv[bb + 1] - p.cu_kv[bb], p.window) : 0;
            const int incl = wave_incl_scan(t);
            const int tot = __builtin_amdgcn_readlane(incl, 63);
            if (start < (acc + tot) * Hu) {
                const bool mine = t > 0 && start >= (acc + incl - t) * Hu && start < (acc + incl) * Hu;
                const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(mine)));
                b = base + src;
                const int tb = __builtin_amdgcn_readlane(t, src);
                const int off = start - (acc + __builtin_amdgcn_readlane(incl - t, src)) * Hu;
                hg = off / tb;
                t0 = off - hg * tb;
                break;
            }
            acc += tot;
        }
    }

    const int G = p.group;
    const int col = lane & 31, g = lane >> 5;
    const bool valid = col < G;
    const bool neg = p.c < 0.f;
    // fp8 cache: the K descale joins the score scale (and the cap's input
    // factor), the V descale multiplies the partial O
    const float dk = KV8 ? p.kv_descale[0] : 1.f;
    const float dv = KV8 ? p.kv_descale[1] : 1.f;
    const float c = fabsf(p.c) * dk;
    const float cap_in2 = p.cap_in2 * dk;
    const int tok_stride = Hkv * D;
    // keys per page window: a range this long starting anywhere fits one
    const int chunk_keys = PAGE_WIN << p.bs_log2;
    uint8_t* mine = smem + w * Tile::BYTES;

    for (int pos = start;;) {
        const int kv_start = p.cu_kv[b];
        const int kv_len = p.cu_kv[b + 1] - kv_start;
        const int klo = decode_klo(kv_len, p.window);
        const int lo_w = p.window > 0 ? max(0, kv_len - p.window) : 0;
        const int nt = (kv_len - klo + 31) >> 5;
        const int t1 = min(nt, t0 + (end - pos));
        const int u = b * Hu + hg;
        const int seg = u + wg;
        if (t0 == 0 && tid == 0) {
            // the unit's last tile lies in workgroup (pos + nt - 1) / C
            p.seg_meta[2 * u] = seg;
            p.seg_meta[2 * u + 1] = (pos + nt - 1) / C - wg + 1;
        }
        const int k0 = klo + 32 * t0;
        const int k1 = min(kv_len, klo + 32 * t1);
        const int hk = hg * HP + hsub;
        const int head = hk * G + col;

        RowsState<D, 1> st;
        st.init();
        {
            const uint16_t* qp = p.q + ((int64_t)b * p.num_heads + head) * D + 8 * g;
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (valid) v = *reinterpret_cast<const u32x4_t*>(qp + 16 * t);
                st.q[0][t] = neg ? neg16x8(v) : v;
            }
        }
        st.lo[0] = lo_w;   // keys before the window are masked
        st.hi[0] = k1;

        const int32_t* table = p.block_table + (int64_t)b * p.mbps;
        const int n_blocks = (kv_len + (1 << p.bs_log2) - 1) >> p.bs_log2;
        const int head_off = hk * D;
        for (int cs = k0; cs < k1; cs += chunk_keys) {
            const int ce = min(k1, cs + chunk_keys);
            const int first = cs >> p.bs_log2;
            fill_page_window(win, table, first, n_blocks, tid, NW * 64);
            __syncthreads();
            // Each wave streams 32-key tiles wt, wt + WPH, ... of the chunk for
            // its kv head through its own LDS slot, with its next tile's loads in
            // flight while it computes.  Chunks are whole tiles except the
            // segment's last, so k1 bounds every tile's rows.
            const int n_t = (ce - cs + 31) >> 5;
            Tile ld;
            auto load = [&](int j) {
                if constexpr (KV8)
                    ld.load(p.k8, p.v8, win, first, j, k1, p.bs_log2, tok_stride, head_off, lane);
                else
                    ld.load(p.k_cache, p.v_cache, win, first, j, k1, p.bs_log2, tok_stride, head_off,
                            lane);
            };
            if (wt < n_t) load(cs + 32 * wt);
            for (int t = wt; t < n_t; t += WPH) {
                const int j = cs + 32 * t;
                ld.store(mine, j, k1, lane);
                __builtin_amdgcn_wave_barrier();
                if (t + WPH < n_t) load(j + 32 * WPH);
                if (j >= lo_w && j + 32 <= k1)
                    tile_step<D, 32, 1, 1, BF16, false, CAP>(st, mine, j, 0, c, cap_in2, p.cap_out);
                else
                    tile_step<D, 32, 1, 1, BF16, true, CAP>(st, mine, j, 0, c, cap_in2, p.cap_out);
                __builtin_amdgcn_wave_barrier();
            }
            __syncthreads();   // the window and the tile slots are free again
        }

        // merge the wave states of each kv head of this segment
        float* red_o = reinterpret_cast<float*>(smem);   // [NW][G][D]
        float* red_m = red_o + NW * G * D;               // [NW][G]
        float* red_l = red_m + NW * G;
        if (valid) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int d = db * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    red_o[(w * G + col) * D + d] = st.o[db][0][r];
                }
            if (g == 0) {
                red_m[w * G + col] = st.m[0];
                red_l[w * G + col] = st.l[0];
            }
        }
        __syncthreads();
        for (int idx = tid; idx < HP * G * D; idx += NW * 64) {
            const int row = idx / D, d = idx % D;   // row = head-in-unit * G + query column
            const int hh = row / G, cc = row - hh * G;
            const int i0 = hh * WPH;                // the head's waves i0 .. i0 + WPH - 1
            float mstar = kNegInf;
            for (int i = i0; i < i0 + WPH; ++i) mstar = fmaxf(mstar, red_m[i * G + cc]);
            float lsum = 0.f, osum = 0.f;
            for (int i = i0; i < i0 + WPH; ++i) {
                const float mi = red_m[i * G + cc];
                const float wgt = (mi == kNegInf) ? 0.f : fast_exp2(mi - mstar);
                lsum += red_l[i * G + cc] * wgt;
                osum += red_o[(i * G + cc) * D + d] * wgt;
            }
            const int64_t slot = (int64_t)seg * (HP * G) + row;
            p.part_o[slot * D + d] = osum * dv;
            if (d == 0) {
                p.part_ml[slot * 2 + 0] = mstar;
                p.part_ml[slot * 2 + 1] = lsum;
            }
        }

        pos += t1 - t0;
        if (pos >= end) break;
        // next unit with tiles (one exists: pos < end <= total)
        t0 = 0;
        if (++hg == Hu) {
            hg = 0;
            do {
                ++b;
            } while (decode_tiles(p.cu_kv[b + 1] - p.cu_kv[b], p.window) == 0);
        }
        __syncthreads();   // the merge's LDS reads precede the next window fill
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(D) void k_decode_combine(DecodeParams p) {
    const int bh = blockIdx.x;
    const int b = bh / p.num_heads;
    const int h = bh - b * p.num_heads;
    const int GP = p.group * p.head_pack;   // partial rows per segment
    const int hg = h / GP;
    const int cc = h - hg * GP;
    const int kv_len = p.cu_kv[b + 1] - p.cu_kv[b];
    int first = 0, n_s = 0;
    if (decode_tiles(kv_len, p.window) > 0) {
        const int u = b * (p.num_kv_heads / p.head_pack) + hg;
        first = p.seg_meta[2 * u];
        n_s = p.seg_meta[2 * u + 1];
    }
    const int d = threadIdx.x;
    float mstar = kNegInf;
    for (int s = 0; s < n_s; ++s)
        mstar = fmaxf(mstar, p.part_ml[((int64_t)(first + s) * GP + cc) * 2]);
    float lsum = 0.f, osum = 0.f;
    for (int s = 0; s < n_s; ++s) {
        const int64_t slot = (int64_t)(first + s) * GP + cc;
        const float ms = p.part_ml[slot * 2];
        const float wgt = (ms == kNegInf) ? 0.f : fast_exp2(ms - mstar);
        lsum += p.part_ml[slot * 2 + 1] * wgt;
        osum += p.part_o[slot * D + d] * wgt;
    }
    const float val = lsum > 0.f ? osum / lsum : 0.f;
    f32x2_t v2 = {val, 0.f};
    uint32_t packed;
    if constexpr (BF16) packed = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2_t));
    else packed = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, f16x2_t));
    p.out[(int64_t)bh * D + d] = (uint16_t)(packed & 0xffffu);
    if (d == 0 && p.lse != nullptr)
        p.lse[bh] = lsum > 0.f ? (mstar + __builtin_log2f(lsum)) * kLn2 : kNegInf;
}

// kv heads per decode unit: 4, 2 or 1, the largest dividing num_kv_heads.
int decode_head_pack(int num_kv_heads) {
    return num_kv_heads % 4 == 0 ? 4 : num_kv_heads % 2 == 0 ? 2 : 1;
}

// Keys a unit's tiles can span for kv lengths up to max_seqlen_kv: with a
// local window W, at most W keys plus up to 31 before them (the tiles start
// 32-key aligned).
int decode_span(int max_seqlen_kv, int window) {
    return window > 0 ? (int)std::min<int64_t>(max_seqlen_kv, (int64_t)window + 31) : max_seqlen_kv;
}

// Upper bound of the tile list's length (every sequence at max_seqlen_kv;
// one tile covers the unit's kv heads).
int64_t decode_tile_bound(int batch, int num_kv_heads, int max_seqlen_kv, int window) {
    const int64_t span = decode_span(max_seqlen_kv, window);
    const int64_t units = (int64_t)batch * (num_kv_heads / decode_head_pack(num_kv_heads));
    return units * ((span + 31) / 32);
}

// Workgroups of the split kernel: with split_tokens the list is cut every
// split_tokens keys (enough workgroups for the longest possible list; the
// ones past its end return at once); by default the grid is `resident`
// workgroups (two per CU), fewer when segments of kDecodeMinSegTiles tiles
// already cover the bound, and at most kDecodeMaxGrid.
int decode_grid(int batch, int num_kv_heads, int max_seqlen_kv, int window, int split_tokens,
                int resident) {
    const int64_t bound = decode_tile_bound(batch, num_kv_heads, max_seqlen_kv, window);
    if (bound <= 0) return 1;
    if (split_tokens > 0) return (int)((bound + split_tokens / 32 - 1) / (split_tokens / 32));
    const int64_t by_min = (bound + kDecodeMinSegTiles - 1) / kDecodeMinSegTiles;
    return (int)std::max<int64_t>(1, std::min<int64_t>({by_min, (int64_t)resident,
                                                         (int64_t)kDecodeMaxGrid}));
}

// Workspace layout: partial slots of one row per query head of the unit,
// one slot per (unit, workgroup) segment, at most units + grid of them
// (part_o, then part_ml), then the per-unit segment records.
DecodeWorkspace decode_workspace(int batch, int num_heads, int num_kv_heads, int head_size,
                                 int max_seqlen_kv, int window, int split_tokens) {
    const int head_units = num_kv_heads / decode_head_pack(num_kv_heads);
    const int64_t units = (int64_t)batch * head_units;
    const int64_t grid = decode_grid(batch, num_kv_heads, max_seqlen_kv, window, split_tokens,
                                     kDecodeMaxGrid);
    const int64_t rows = (units + grid) * (num_heads / head_units);
    DecodeWorkspace ws;
    ws.ml_off = (size_t)(((rows * head_size * 4 + 255) / 256) * 256);
    ws.meta_off = ws.ml_off + (size_t)(((rows * 2 * 4 + 255) / 256) * 256);
    ws.bytes = ws.meta_off + (size_t)(units * 2 * 4);
    return ws;
}

// Compute units of the current device (looked up once per device).
hipError_t cu_count(int* out) {
    static std::atomic<int> known[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int v = known[dev].load(std::memory_order_acquire);
        if (v > 0) {
            *out = v;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    n = std::max(1, n);
    if (dev >= 0 && dev < 64) known[dev].store(n, std::memory_order_release);
    *out = n;
    return hipSuccess;
}

// Split partials of the allocation-free decode entry point: one array per
// GPU, created with the code object on each device and held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept per device ordinal.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
    constexpr int kSlots = 64;
    static std::atomic<void*> addr[kSlots];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kSlots) {
        void* known = addr[dev].load(std::memory_order_acquire);
        if (known != nullptr) {
            *ptr = known;
            return hipSuccess;
        }
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    if (dev >= 0 && dev < kSlots) addr[dev].store(p, std::memory_order_release);
    *ptr = p;
    return hipSuccess;
}

namespace {

template <int D, int NW, bool BF16, bool CAP, bool KV8>
hipError_t launch_decode_cfg(const DecodeParams& p, hipStream_t s) {
    constexpr int lds = DecodeLayout<D, NW, BF16, KV8>::LDS_BYTES;
    // The dynamic-LDS limit is a per-device function attribute: set it once
    // on each device this launcher runs on (one bit per device ordinal;
    // ordinals past 63 set it on every launch).
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (bit == 0 || (attr_set.load(std::memory_order_acquire) & bit) == 0) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_paged_decode<D, NW, BF16, CAP, KV8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit, std::memory_order_acq_rel);
    }
    if (p.grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_paged_decode<D, NW, BF16, CAP, KV8>), dim3((unsigned)p.grid), dim3(NW * 64),
                       lds, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_decode_combine<D, BF16>), dim3((unsigned)(p.batch * p.num_heads)),
                       dim3(D), 0, s, p);
    return hipGetLastError();
}

}  // namespace

template <int D, bool BF16, bool KV8>
hipError_t launch_decode_cap(const DecodeParams& p, hipStream_t s) {
    return p.cap_out > 0.f ? launch_decode_cfg<D, 4, BF16, true, KV8>(p, s)
                           : launch_decode_cfg<D, 4, BF16, false, KV8>(p, s);
}

template <bool KV8>
hipError_t launch_decode_kv(const DecodeParams& p, int head_size, bool bf16, hipStream_t s) {
    if (head_size == 128)
        return bf16 ? launch_decode_cap<128, true, KV8>(p, s) : launch_decode_cap<128, false, KV8>(p, s);
    if (head_size == 64)
        return bf16 ? launch_decode_cap<64, true, KV8>(p, s) : launch_decode_cap<64, false, KV8>(p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode(const DecodeParams& p, int head_size, bool bf16, hipStream_t s) {
    return p.k8 != nullptr ? launch_decode_kv<true>(p, head_size, bf16, s)
                           : launch_decode_kv<false>(p, head_size, bf16, s);
}

}  // namespace attn
