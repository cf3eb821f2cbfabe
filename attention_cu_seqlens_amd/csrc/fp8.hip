// Dense varlen fp8 e4m3 attention with a column-major V on gfx950.
//
// The fp8 path of the pytorch commit "[FlexAttention] Enforce Q,K,V memory
// layouts for fp8 flex attention to avoid perf degradation": Q and K are
// row-major, V is column-major ([Hkv, D, total_kv], key-contiguous), which is
// the layout the P.V product wants for its V operand (commit message,
// Context; _enforce_mem_layouts).  Here that V tile is a plain 16-byte copy
// into LDS.
//
// Both products use the 32x32x64 fp8 MFMA (format E4M3 for both operands,
// no block scale).  S^T = K.Q^T as in the 16-bit kernels; for P^T.V the
// scores of two 32-key blocks form one 64-key operand.  A lane's 32 score
// registers of those blocks are rows {8b + 4g + e} of each block; the K tile
// rows are read through a permutation so that those 32 registers hold keys
// 32g .. 32g+31 of the 64-key group, which makes each lane's V^T operand 32
// consecutive bytes of one V^T row.
//
// Numerics: scores = (scale * dq * dk) * (q8 . k8) in fp32; online softmax in
// fp32; P is rounded to e4m3 (nearest even) for the P.V product and the row
// normaliser l is summed from those rounded values, so O = dv * (P8 . V8) / l
// is a convex combination of V rows.

#include "device_common.h"
#include "kernels.h"

namespace attn {

namespace {

__device__ __forceinline__ f32x16_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

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

// K tile row read by A-operand lane row j of 32-key block kb = 2*gp + a.
__device__ __forceinline__ int fp8_krow(int kb, int j) {
    const int gp = kb >> 1, a = kb & 1;
    return 64 * gp + 16 * a + 32 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3);
}
__device__ __forceinline__ int fp8_kswz(int row) { return (row & 3) | (((row >> 5) & 1) << 2); }

constexpr int D8 = 128;     // head size (bytes per row)
constexpr int BN8 = 128;    // keys per tile

// LDS: K [BN8][128 B] (chunk c at c ^ fp8_kswz(row)), then Vt [128][BN8 B]
// (key-contiguous rows, chunk c at c ^ (d & 7)).
template <int NT>
struct DenseTile8 {
    static constexpr int K_BYTES = BN8 * D8;
    static constexpr int V_BYTES = D8 * BN8;
    static constexpr int BYTES = K_BYTES + V_BYTES;
    static constexpr int KPT = (K_BYTES / 16) / NT;
    static constexpr int VPT = (V_BYTES / 16) / NT;
    static_assert(KPT >= 1 && VPT >= 1, "tile too small for the workgroup");
    u32x4_t kreg[KPT];
    u32x4_t vreg[VPT];

    // keys [j0, j0 + BN8) of a sequence starting at global key kv_start
    // (kv_len >= 1).  Loads past kv_len read a valid row / chunk of the same
    // sequence and are zeroed by store(), so the loads issue back to back.
    __device__ __forceinline__ void load(const uint8_t* __restrict__ k, const uint8_t* __restrict__ vt,
                                         int64_t total_kv, int kv_start, int j0, int kv_len,
                                         int k_tok_stride, int k_head_off, int64_t v_head_base,
                                         bool v_aligned, int tid) {
        const int last = kv_len - 1;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            const int row = idx >> 3, c = idx & 7;
            const int key = min(j0 + row, last);
            kreg[i] = *reinterpret_cast<const u32x4_t*>(
                k + (int64_t)(kv_start + key) * k_tok_stride + k_head_off + c * 16);
        }
        if (v_aligned) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = tid + i * NT;
                const int d = idx >> 3, c = idx & 7;
                const int key0 = min(j0 + c * 16, last & ~15);
                vreg[i] = *reinterpret_cast<const u32x4_t*>(
                    vt + v_head_base + (int64_t)d * total_kv + kv_start + key0);
            }
        } else {
            // unaligned varlen layout: byte loads of the valid keys only
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = tid + i * NT;
                const int d = idx >> 3, c = idx & 7;
                const int key0 = j0 + c * 16;
                const uint8_t* src = vt + v_head_base + (int64_t)d * total_kv + kv_start + key0;
                uint32_t wds[4] = {0u, 0u, 0u, 0u};
                const int n = kv_len - key0;
                for (int bI = 0; bI < 16 && bI < n; ++bI)
                    wds[bI >> 2] |= (uint32_t)src[bI] << (8 * (bI & 3));
                vreg[i] = u32x4_t{wds[0], wds[1], wds[2], wds[3]};
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t* lds, int j0, int kv_len, int tid) const {
        const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            const int row = idx >> 3, c = idx & 7;
            const u32x4_t v = (j0 + row < kv_len) ? kreg[i] : zero;
            *reinterpret_cast<u32x4_t*>(lds + row * D8 + ((c ^ fp8_kswz(row)) << 4)) = v;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + i * NT;
            const int d = idx >> 3, c = idx & 7;
            const int n = kv_len - (j0 + c * 16);   // valid keys in this 16-key chunk
            u32x4_t v = vreg[i];
            if (n < 16) {
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const int keep = n - 4 * wd;
                    const uint32_t msk = keep >= 4 ? 0xffffffffu
                                       : keep <= 0 ? 0u
                                                   : (0xffffffffu >> (32 - 8 * keep));
                    v[wd] &= msk;
                }
            }
            *reinterpret_cast<u32x4_t*>(lds + K_BYTES + d * BN8 + ((c ^ (d & 7)) << 4)) = v;
        }
    }
};

template <int QB>
struct Fp8Rows {
    i32x8_t q[QB][2];          // Q^T operand: dims 64t + 32g .. +31 per lane-half
    f32x16_t o[4][QB];         // O^T accumulators (P8 . V8, unscaled)
    float m[QB], l[QB];
    int lo[QB], hi[QB];
};

template <int QB, bool MASKED>
__device__ __forceinline__ void fp8_tile_step(Fp8Rows<QB>& st, const uint8_t* lds, int j0,
                                              float c) {
    const uint8_t* lk = lds;
    const uint8_t* lv = lds + BN8 * D8;
    const int lane = lane_id();
    const int col = lane & 31, g = lane >> 5;

    f32x16_t s[4][QB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16_t{};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int row = fp8_krow(kb, col);
            const uint8_t* rp = lk + row * D8;
            const int c0 = 4 * t + 2 * g;
            const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(rp + ((c0 ^ fp8_kswz(row)) << 4));
            const u32x4_t hi4 =
                *reinterpret_cast<const u32x4_t*>(rp + (((c0 + 1) ^ fp8_kswz(row)) << 4));
            const i32x8_t a = {(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                               (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma_fp8(a, st.q[qb][t], s[kb][qb]);
        }

    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (MASKED) {
                    // key held by register r of block kb for this lane
                    const int key = j0 + 64 * (kb >> 1) + 32 * g + 16 * (kb & 1) + r;
                    if (!(key >= st.lo[qb] && key < st.hi[qb])) s[kb][qb][r] = kNegInf;
                }
                mx[qb] = fmaxf(mx[qb], s[kb][qb][r]);
            }

    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mx[qb] = fmaxf(mx[qb], xor32(mx[qb]));
        mx[qb] = (mx[qb] == kNegInf) ? kNegInf : mx[qb] * c;
        need |= mx[qb] > st.m[qb] + kRescaleSlack;
    }
    if (__any(need)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mnew = fmaxf(st.m[qb], mx[qb]);
            const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(st.m[qb] - mnew);
            st.m[qb] = mnew;
            st.l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) st.o[db][qb] *= alpha;
        }
    }

    float rs[QB];
    i32x8_t pb[2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        rs[qb] = 0.f;
        const float nm = (st.m[qb] == kNegInf) ? 0.f : -st.m[qb];
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
#pragma unroll
            for (int wd = 0; wd < 8; ++wd) {
                const int kb = 2 * gp + (wd >> 2);
                const int r0 = 4 * (wd & 3);
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sv = s[kb][qb][r0 + e];
                    pv[e] = fast_exp2(__builtin_fmaf(sv, c, nm));
                    if constexpr (MASKED) pv[e] = (sv == kNegInf) ? 0.f : pv[e];
                }
                int packed = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
                packed = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], packed, true);
                pb[gp][qb][wd] = packed;
                const f32x2_t back_lo = __builtin_amdgcn_cvt_pk_f32_fp8(packed, false);
                const f32x2_t back_hi = __builtin_amdgcn_cvt_pk_f32_fp8(packed, true);
                rs[qb] += (back_lo.x + back_lo.y) + (back_hi.x + back_hi.y);
            }
        }
        st.l[qb] += rs[qb] + xor32(rs[qb]);
    }

#pragma unroll
    for (int gp = 0; gp < 2; ++gp)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int d = db * 32 + col;
            const uint8_t* rp = lv + d * BN8;
            const int c0 = 4 * gp + 2 * g;
            const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(rp + ((c0 ^ (d & 7)) << 4));
            const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(rp + (((c0 + 1) ^ (d & 7)) << 4));
            const i32x8_t a = {(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                               (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) st.o[db][qb] = mfma_fp8(a, pb[gp][qb], st.o[db][qb]);
        }
}

}  // namespace

template <int QB, int NW>
__global__ __launch_bounds__(NW * 64) void k_fp8_prefill(Fp8Params p) {
    constexpr int NT = NW * 64;
    constexpr int BM = NW * QB * 32;
    using Tile = DenseTile8<NT>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * Tile::BYTES];
    __shared__ int wave_range[2][NW];

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
    const float dq = p.descale[0], dk = p.descale[1], dv = p.descale[2];
    const float c_signed = p.scale * dq * dk * kLog2e;
    const bool neg = c_signed < 0.f;
    const float c = fabsf(c_signed);

    const int tid = threadIdx.x;
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 31, g = lane >> 5;

    Fp8Rows<QB> st;
    int tok[QB], head[QB];
    bool valid[QB];
    int my_lo = 0x7fffffff, my_hi = -0x7fffffff, my_lo_max = -0x7fffffff, my_hi_min = 0x7fffffff;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        st.m[qb] = kNegInf;
        st.l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db) st.o[db][qb] = f32x16_t{};
        const int r = (w * QB + qb) * 32 + col;
        tok[qb] = tok0 + (r >> p.pack_log2);
        head[qb] = h0 + (r & ((1 << p.pack_log2) - 1));
        valid[qb] = tok[qb] < q_len;
        const uint8_t* qp = p.q + ((int64_t)(q_start + tok[qb]) * p.num_heads + head[qb]) * D8 + 32 * g;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            i32x8_t v = {};
            if (valid[qb]) {
                const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(qp + 64 * t);
                const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(qp + 64 * t + 16);
                v = i32x8_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                            (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                if (neg) v ^= (int)0x80808080u;   // apply a negative scale to -q
            }
            st.q[qb][t] = v;
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
    kv_begin &= ~15;
    const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + BN8 - 1) / BN8 : 0;

    const int k_tok_stride = p.num_kv_heads * D8;
    const int k_head_off = hk * D8;
    const int64_t v_head_base = (int64_t)hk * D8 * p.total_kv;
    const bool v_aligned = ((p.total_kv & 15) == 0) && ((kv_start & 15) == 0);
    Tile ld;
    if (n_tiles > 0) {
        ld.load(p.k, p.vt, p.total_kv, kv_start, kv_begin, kv_len, k_tok_stride, k_head_off,
                v_head_base, v_aligned, tid);
        ld.store(smem, kv_begin, kv_len, tid);
    }
    __syncthreads();
    for (int it = 0; it < n_tiles; ++it) {
        const int j = kv_begin + it * BN8;
        const uint8_t* cur = smem + (it & 1) * Tile::BYTES;
        const bool has_next = it + 1 < n_tiles;
        if (has_next)
            ld.load(p.k, p.vt, p.total_kv, kv_start, j + BN8, kv_len, k_tok_stride, k_head_off,
                    v_head_base, v_aligned, tid);
        if (w_any && j < w_hi && j + BN8 > w_lo) {
            if (j >= w_lo_max && j + BN8 <= w_hi_min)
                fp8_tile_step<QB, false>(st, cur, j, c);
            else
                fp8_tile_step<QB, true>(st, cur, j, c);
        }
        if (has_next) ld.store(smem + ((it + 1) & 1) * Tile::BYTES, j + BN8, kv_len, tid);
        __syncthreads();
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        if (!valid[qb]) continue;
        const int64_t row = (int64_t)(q_start + tok[qb]) * p.num_heads + head[qb];
        f32x16_t o_db[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) o_db[db] = st.o[db][qb] * dv;
        store_row<D8, true>(o_db, st.l[qb], p.out + row * D8);
        if (p.lse != nullptr && g == 0)
            p.lse[row] = st.l[qb] > 0.f ? (st.m[qb] + __builtin_log2f(st.l[qb])) * kLn2 : kNegInf;
    }
}

hipError_t launch_fp8_prefill(const Fp8Params& p0, int head_size, int max_seqlen_q,
                              hipStream_t s) {
    if (head_size != D8) return hipErrorInvalidValue;
    constexpr int QB = 1, NW = 8;
    constexpr int BM = NW * QB * 32;
    Fp8Params p = p0;
    const int tokens_per_tile = BM >> p.pack_log2;
    p.n_qtiles = (max_seqlen_q + tokens_per_tile - 1) / tokens_per_tile;
    const int64_t grid = 8 * tiles_per_xcd(p.batch, p.n_head_groups, p.total_q, max_seqlen_q,
                                           tokens_per_tile);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_fp8_prefill<QB, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace attn
