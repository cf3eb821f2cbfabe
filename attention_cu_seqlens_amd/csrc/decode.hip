// Paged GQA decode (one query token per sequence) for 16-bit dtypes on gfx950.
//
// Split-KV: workgroup (sequence b, kv head hk, split s) streams keys
// [s*split_tokens, (s+1)*split_tokens) of the paged cache.  Its NW waves take
// interleaved 32-key blocks of each BN = 32*NW key tile, each with its own
// online-softmax state for the G = Hq/Hkv query heads of the group (the 32
// query columns of the MFMA, G of them live).  The waves merge in LDS at the
// end and the workgroup writes one partial (unnormalised O, running max m,
// sum l) per query head.  A second kernel merges the splits with the same
// logsumexp rule; its LSE output is the "OUTPUT_LOGSUMEXP" quantity of the
// FlexAttention kernel options shown in the blt issue "Cross Attention does
// not work on CPU and older GPUs".
//
// The grid is sized from max_seqlen_kv on the host (no device->host sync);
// splits past a sequence's end exit at once and the merge kernel derives
// each sequence's split count from its own length.

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

template <int D, int NW, bool BF16, bool CAP, bool KV8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_paged_decode(DecodeParams p) {
    using L = DecodeLayout<D, NW, BF16, KV8>;
    using Tile = typename L::Tile;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int* win = reinterpret_cast<int*>(smem + L::WIN_OFF);

    // Split index outermost: workgroup i runs on XCD i % 8, so consecutive
    // workgroups are different (sequence, kv head) units of the same split
    // and every XCD gets an equal share of each split index.  (Split-fastest
    // order piles the low split indices, which every sequence has, onto the
    // XCDs they map to whenever the split count is a multiple of 8.)
    const int units = p.batch * p.num_kv_heads;
    const int s = blockIdx.x / units;
    const int unit = blockIdx.x - s * units;
    const int hk = unit % p.num_kv_heads;
    const int b = unit / p.num_kv_heads;
    const int kv_start = p.cu_kv[b];
    const int kv_len = p.cu_kv[b + 1] - kv_start;
    // The splits tile the keys from window_base (0 without a local window):
    // a window keeps the sequence's last p.window keys, lo_w on; the grid
    // starts at lo_w rounded down to 32 keys (tiles stay 32-key aligned) and
    // the keys before lo_w are masked.
    const int lo_w = p.window > 0 ? max(0, kv_len - p.window) : 0;
    const int k0 = (lo_w & ~31) + s * p.split_tokens;
    if (k0 >= kv_len) return;
    const int k1 = min(kv_len, k0 + p.split_tokens);
    const bool neg = p.c < 0.f;
    // fp8 cache: the K descale joins the score scale (and the cap's input
    // factor), the V descale multiplies the partial O
    const float dk = KV8 ? p.kv_descale[0] : 1.f;
    const float dv = KV8 ? p.kv_descale[1] : 1.f;
    const float c = fabsf(p.c) * dk;
    const float cap_in2 = p.cap_in2 * dk;

    const int tid = threadIdx.x;
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 31, g = lane >> 5;
    const int G = p.group;
    const bool valid = col < G;
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
    const int first = k0 >> p.bs_log2;
    fill_page_window(win, table, first, n_blocks, tid, NW * 64);
    __syncthreads();

    // Each wave streams 32-key tiles w, w + NW, ... of the split through its
    // own LDS slot, with its next tile's loads in flight while it computes.
    const int tok_stride = p.num_kv_heads * D;
    const int head_off = hk * D;
    const int n_t = (k1 - k0 + 31) >> 5;
    // tiles wholly below the window hold no visible key: start past them
    const int t_first = lo_w > k0 ? (lo_w - k0) >> 5 : 0;
    uint8_t* mine = smem + w * Tile::BYTES;
    Tile ld;
    auto load = [&](int j) {
        if constexpr (KV8)
            ld.load(p.k8, p.v8, win, first, j, k1, p.bs_log2, tok_stride, head_off, lane);
        else
            ld.load(p.k_cache, p.v_cache, win, first, j, k1, p.bs_log2, tok_stride, head_off, lane);
    };
    if (t_first + w < n_t) load(k0 + 32 * (t_first + w));
    for (int t = t_first + w; t < n_t; t += NW) {
        const int j = k0 + 32 * t;
        ld.store(mine, j, k1, lane);
        __builtin_amdgcn_wave_barrier();
        if (t + NW < n_t) load(j + 32 * NW);
        if (j >= lo_w && j + 32 <= k1)
            tile_step<D, 32, 1, 1, BF16, false, CAP>(st, mine, j, 0, c, cap_in2, p.cap_out);
        else
            tile_step<D, 32, 1, 1, BF16, true, CAP>(st, mine, j, 0, c, cap_in2, p.cap_out);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // merge the NW wave states of this split
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
    for (int idx = tid; idx < G * D; idx += NW * 64) {
        const int cc = idx / D, d = idx % D;
        float mstar = kNegInf;
#pragma unroll
        for (int i = 0; i < NW; ++i) mstar = fmaxf(mstar, red_m[i * G + cc]);
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const float mi = red_m[i * G + cc];
            const float wgt = (mi == kNegInf) ? 0.f : fast_exp2(mi - mstar);
            lsum += red_l[i * G + cc] * wgt;
            osum += red_o[(i * G + cc) * D + d] * wgt;
        }
        const int64_t slot = ((int64_t)b * p.num_heads + hk * G + cc) * p.max_splits + s;
        p.part_o[slot * D + d] = osum * dv;
        if (d == 0) {
            p.part_ml[slot * 2 + 0] = mstar;
            p.part_ml[slot * 2 + 1] = lsum;
        }
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(D) void k_decode_combine(DecodeParams p) {
    const int bh = blockIdx.x;
    const int b = bh / p.num_heads;
    const int kv_len = p.cu_kv[b + 1] - p.cu_kv[b];
    const int lo_w = p.window > 0 ? max(0, kv_len - p.window) : 0;
    const int n_s = (kv_len - (lo_w & ~31) + p.split_tokens - 1) / p.split_tokens;
    const int d = threadIdx.x;
    const int64_t base = (int64_t)bh * p.max_splits;
    float mstar = kNegInf;
    for (int s = 0; s < n_s; ++s) mstar = fmaxf(mstar, p.part_ml[(base + s) * 2]);
    float lsum = 0.f, osum = 0.f;
    for (int s = 0; s < n_s; ++s) {
        const float ms = p.part_ml[(base + s) * 2];
        const float wgt = (ms == kNegInf) ? 0.f : fast_exp2(ms - mstar);
        lsum += p.part_ml[(base + s) * 2 + 1] * wgt;
        osum += p.part_o[(base + s) * D + d] * wgt;
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

// Automatic split size: the smallest power of two (>= 256 keys) that keeps the
// grid at no more than 4096 workgroups, i.e. about 8 rounds of the two
// resident workgroups per CU.  Fewer, longer workgroups pay the per-workgroup
// start (block ids, first tile from HBM) less often; the paged GQA decode
// workload (64 sequences, kv 1024-32768, 8 kv heads) measured 5.8-6.0 TB/s at
// 4096 keys per split against 5.1 at 512 and 5.5 at 1024.
// Keys a split grid must cover for kv lengths up to max_seqlen_kv: with a
// local window W, at most W keys plus up to 31 before them (the grid starts
// 32-key aligned).
int decode_span(int max_seqlen_kv, int window) {
    return window > 0 ? (int)std::min<int64_t>(max_seqlen_kv, (int64_t)window + 31) : max_seqlen_kv;
}

int decode_split_tokens(int batch, int num_kv_heads, int max_seqlen_kv, int requested) {
    if (requested > 0) return requested;
    const int64_t units = (int64_t)batch * num_kv_heads;
    int st = 256;
    while (st < 8192 && units * ((max_seqlen_kv + st - 1) / st) > 4096) st *= 2;
    return st;
}

size_t decode_workspace_bytes(int batch, int num_heads, int head_size, int max_seqlen_kv,
                              int split_tokens) {
    const int64_t splits = max_seqlen_kv > 0 ? (max_seqlen_kv + split_tokens - 1) / split_tokens : 1;
    const int64_t rows = (int64_t)batch * num_heads * splits;
    const int64_t o_bytes = ((rows * head_size * 4 + 255) / 256) * 256;
    return (size_t)(o_bytes + rows * 2 * 4);
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
    const int64_t grid = (int64_t)p.batch * p.num_kv_heads * p.max_splits;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_paged_decode<D, NW, BF16, CAP, KV8>), dim3((unsigned)grid), dim3(NW * 64),
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
