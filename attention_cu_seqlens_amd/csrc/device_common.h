// Device building blocks shared by the gfx950 attention kernels.
//
// Formulation.  Every kernel computes the transposed products
//     S^T = K . Q^T        (rows = keys, columns = queries)
//     O^T += V^T . P^T     (rows = head dims, columns = queries)
// with the 32x32 MFMA.  In the 32x32 accumulator layout lane l owns column
// l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 of register r, so each lane holds
// one query's scores for 16 keys per 32-key block: the row max and row sum of
// the online softmax are mostly in-lane (one exchange with lane l ^ 32), the
// per-query rescale of O^T is a per-lane scalar, and the probabilities feed
// the P^T operand of the second product straight from the score registers.
// The price is that the V operand must be contiguous along the key axis --
// the column-major V that the FlexAttention fp8 commit ("[FlexAttention]
// Enforce Q,K,V memory layouts for fp8 flex attention...", Context) asks
// for.  The paged cache holds V token-major, so the tile loader transposes V
// in registers on its way into LDS.
//
// Only operand consistency matters for an MFMA contraction: element e of
// lane-half g in the A operand is multiplied with element e of lane-half g in
// the B operand.  The loaders below place matching (key, dim) pairs at
// matching (half, element) positions; they do not depend on the hardware's
// internal k order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// 32x32x16 MFMA on 8 packed 16-bit values per lane (4 dwords).
template <bool BF16>
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// Two fp32 values -> two 16-bit values (round to nearest even), low first.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    if constexpr (BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Score cap (softcap c > 0) in the kernels' log2 domain: from the raw
// product s, c * tanh(|scale| * s / c) * log2(e) = out * (1 - 2 / (1 + 2^(s * in2)))
// with in2 = 2 * log2(e) * |scale| / c and out = c * log2(e).  2^(.)
// overflows to +inf for large arguments (exactly +out) and underflows to 0
// (exactly -out); a masked score (-inf) stays -inf.
__device__ __forceinline__ float cap_score(float s, float in2, float out) {
    const float e = fast_exp2(s * in2);
    const float t = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + e), 1.f);
    return s == kNegInf ? kNegInf : out * t;
}

// Exchange with lane ^ 32 (the other half of a 32-wide MFMA column).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Both halves of x: v_permlane32_swap (a VALU op, no LDS round trip unlike
// a ds_bpermute shuffle) exchanges lanes 32-63 of its first register with
// lanes 0-31 of its second.  Given two copies of x, the first then holds
// lanes 0-31 of x in both halves and the second lanes 32-63, so
// op(first, second) pairs each lane with lane ^ 32; max and + commute, so
// both lanes of a pair get the same bits.  Written as asm (both registers
// are outputs): the compiler's builtin for it merged the two results into
// one.  The s_nop gives the two wait states a permlane needs after a VALU
// write of its operands.
__device__ __forceinline__ f32x2_t pair_halves(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return f32x2_t{a, b};
}
// max / sum of x over the lane pair (l, l ^ 32), the same value in both lanes
__device__ __forceinline__ float pair_max(float x) {
    const f32x2_t h = pair_halves(x);
    return fmaxf(h.x, h.y);
}
__device__ __forceinline__ float pair_sum(float x) {
    const f32x2_t h = pair_halves(x);
    return h.x + h.y;
}

// Lane moves within rows of 16 lanes (DPP, GFX9 encodings): quad_perm
// [1,0,3,2] and [2,3,0,1], the half-row and row mirrors, and row_shr:s
// (0x110 + s; lanes with no source lane in their row read 0).  A DPP move
// runs on the VALU, with no LDS round trip as a lane shuffle has.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };
template <int CTRL>
__device__ __forceinline__ int dpp_move(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}

// Reductions over the 64 lanes (every lane active); the result is
// wave-uniform.  Within a row the moves pair lanes i^1, i^2, the two
// halves and the two 8-lane halves' mirrors, so every lane ends with its
// row's extreme; the four rows are combined on the scalar unit.
__device__ __forceinline__ int wave_min(int x) {
    x = min(x, dpp_move<kDppXor1>(x));
    x = min(x, dpp_move<kDppXor2>(x));
    x = min(x, dpp_move<kDppHalfMirror>(x));
    x = min(x, dpp_move<kDppMirror>(x));
    return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
// Inclusive prefix sum over the 64 lanes: a Hillis-Steele scan inside each
// row (shifts 1, 2, 4, 8), then each row adds the totals of the rows below.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += dpp_move<0x111>(x);
    x += dpp_move<0x112>(x);
    x += dpp_move<0x114>(x);
    x += dpp_move<0x118>(x);
    const int r0 = __builtin_amdgcn_readlane(x, 15);
    const int r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47);
    const int row = lane_id() >> 4;
    return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// The token ranges of one sequence in the packed query and key arrays.
struct SeqSpan {
    int q_start, q_len, kv_start, kv_len;
};

// Work item k of XCD `xcd` (workgroup i runs on XCD i % 8, k = i / 8) ->
// (sequence b, head group hg, query tile qt), for query tiles of `tt` tokens,
// and the sequence's spans.  Units u = b * n_hg + hg are dealt to XCDs
// round-robin (XCD x owns units x, x + 8, ...); an XCD walks its units in
// order and each unit's query tiles longest first, so the tiles that share
// one K/V stream run together on one XCD and its L2.  Only existing tiles get
// a work item, so short sequences leave no idle workgroups behind; returns
// false past the XCD's last tile.  The cu_seqlens entries of both sides are
// read in one round trip.  Wave-uniform; every wave of a workgroup computes
// the same.
__device__ __forceinline__ bool map_tile(const int32_t* cu_q, const int32_t* cu_kv, int batch,
                                         int n_hg, int tt, int xcd, int k, int& b, int& hg,
                                         int& qt, SeqSpan& sp) {
    const int units = batch * n_hg;
    const int lane = lane_id();
    int base = 0;   // tiles of the chunks before this one
    for (int m0 = 0; xcd + 8 * m0 < units; m0 += 64) {
        const int u = xcd + 8 * (m0 + lane);
        int q0 = 0, q1 = 0, k0 = 0, k1 = 0;
        if (u < units) {
            const int bb = u / n_hg;
            q0 = cu_q[bb];
            q1 = cu_q[bb + 1];
            k0 = cu_kv[bb];
            k1 = cu_kv[bb + 1];
        }
        const int t = (q1 - q0 + tt - 1) / tt;
        const int incl = wave_incl_scan(t);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (k < base + total) {
            const bool mine = k >= base + incl - t && k < base + incl;
            const uint64_t who = __ballot(mine);
            const int src = __builtin_amdgcn_readfirstlane(__builtin_ctzll(who));
            const int uu = __builtin_amdgcn_readlane(u, src);
            const int first = __builtin_amdgcn_readlane(incl - t, src);
            const int tu = __builtin_amdgcn_readlane(t, src);
            b = uu / n_hg;
            hg = uu - b * n_hg;
            qt = tu - 1 - (k - base - first);
            sp.q_start = __builtin_amdgcn_readlane(q0, src);
            sp.q_len = __builtin_amdgcn_readlane(q1, src) - sp.q_start;
            sp.kv_start = __builtin_amdgcn_readlane(k0, src);
            sp.kv_len = __builtin_amdgcn_readlane(k1, src) - sp.kv_start;
            return true;
        }
        base += total;
    }
    return false;
}

// Workgroups per XCD that cover every query tile of tt tokens: each XCD owns
// at most ceil(n_hg / 8) units of any one sequence, and a sequence of len
// tokens has ceil(len / tt) <= (len + tt - 1) / tt tiles.
inline int64_t tiles_per_xcd(int batch, int n_hg, int total_q, int max_seqlen_q, int tt) {
    const int64_t units = (int64_t)batch * n_hg;
    const int64_t by_len = ((units + 7) / 8) * ((max_seqlen_q + tt - 1) / tt);
    const int64_t by_total = (int64_t)((n_hg + 7) / 8) * (((int64_t)total_q + (int64_t)batch * (tt - 1)) / tt);
    return by_len < by_total ? by_len : by_total;
}

// Binary searches over a non-decreasing int32 array a[0..n).
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

__device__ __forceinline__ int wave_max(int x) {
    x = max(x, dpp_move<kDppXor1>(x));
    x = max(x, dpp_move<kDppXor2>(x));
    x = max(x, dpp_move<kDppHalfMirror>(x));
    x = max(x, dpp_move<kDppMirror>(x));
    return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Bits 2 and 3 of a key index swapped.  The accumulator rows a lane feeds to
// one 16-key P^T step are keys {4g..4g+3} and {8+4g..8+4g+3}; storing key k at
// V^T slot swap23(k) makes those 8 keys one contiguous 16-byte LDS read.
__device__ __forceinline__ int swap23(int k) {
    return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// LDS row pitches: one extra 16-byte chunk per row shifts consecutive rows by
// one bank group, so the 8 (or 16) lanes that read one 16-byte chunk of 8
// (16) consecutive rows hit distinct banks, and every fragment read is a
// per-lane base plus a compile-time offset.
template <int D> constexpr int k_pitch() { return D * 2 + 16; }
template <int BN> constexpr int vt_pitch() { return BN * 2 + 16; }

// ---------------------------------------------------------------------------
// Block-table window.  The physical block ids of a key range are staged in
// LDS once (all loads in flight together), so the K/V loads of every tile
// find their page with an LDS read instead of a dependent global load.
// A window holds PAGE_WIN + 1 ids starting at logical block `first`; a key
// range of PAGE_WIN * block_size keys starting anywhere fits in it.
// ---------------------------------------------------------------------------
constexpr int PAGE_WIN = 512;

template <bool STREAM>
__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
    if constexpr (STREAM)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    else
        return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ void fill_page_window(int* win, const int32_t* __restrict__ table,
                                                 int first, int n_blocks, int tid, int nt) {
    for (int i = tid; i <= PAGE_WIN; i += nt) {
        const int p = first + i;
        win[i] = p < n_blocks ? table[p] : 0;
    }
}

// ---------------------------------------------------------------------------
// Paged K/V tile loader for 16-bit dtypes.
//
// A tile is BN consecutive keys of one sequence and one kv head.  LDS gets
//   K  [BN][D]  16-bit, row = key, pitch k_pitch<D>()
//   Vt [D][BN]  16-bit, row = dim, key k at slot swap23(k), pitch vt_pitch<BN>()
// Keys at or past kv_len are zero-filled (the cache may hold NaN there).
// Loads are unconditional: a row past kv_len is read from a valid row of the
// same sequence and zeroed when stored, so a tile's loads issue back to back.
// K is moved in 16-byte chunks (16 lanes cover one 256-byte row).  V moves in
// units of 4 keys x 8 dims, transposed in registers (4 rows x 4 dwords -> 8
// dim rows x 2 dwords) and written as eight 8-byte stores; units are numbered
// key-quad fastest so the 8-byte stores of neighbouring lanes are contiguous.
// STREAM marks the loads non-temporal (decode reads each byte once; prefill
// re-reads K/V across query tiles and keeps them cacheable).
// ---------------------------------------------------------------------------
template <int D, int BN, int NT, bool STREAM>
struct PagedTile16 {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per key row
    static constexpr int QPT = BN / 4;                // key quads per tile
    static constexpr int NV = QPT * CPR;              // V units per tile
    static constexpr int NK = BN * CPR;               // K chunks per tile
    // SPLIT: fewer V units than threads -- threads [0, NV) take one V unit
    // each and the others share the K chunks; otherwise every thread takes
    // NV/NT V units and NK/NT K chunks.  Either way each thread issues the
    // same number of 16-byte loads.
    static constexpr bool SPLIT = NV < NT;
    static constexpr int KT = SPLIT ? NT - NV : NT;   // threads loading K
    static constexpr int VPT = SPLIT ? 1 : NV / NT;
    static constexpr int KPT = NK / KT;
    static_assert(SPLIT ? (NV % 64 == 0 && NK % KT == 0) : (NV % NT == 0 && NK % NT == 0),
                  "tile does not divide over the workgroup");
    static_assert(!SPLIT || KPT == 4 * VPT, "unbalanced split");
    static constexpr int KP = k_pitch<D>();
    static constexpr int VP = vt_pitch<BN>();
    static constexpr int K_BYTES = BN * KP;
    static constexpr int V_BYTES = D * VP;
    static constexpr int BYTES = K_BYTES + V_BYTES;

    u32x4_t kreg[KPT];
    u32x4_t vreg[VPT][4];

    __device__ __forceinline__ bool does_k(int tid) const { return !SPLIT || tid >= NV; }
    __device__ __forceinline__ bool does_v(int tid) const { return !SPLIT || tid < NV; }
    __device__ __forceinline__ int k_index(int tid, int i) const {
        return (SPLIT ? tid - NV : tid) + i * KT;
    }

    // Issue the global loads for keys [j0, j0 + BN) of one sequence
    // (kv_len >= 1).  win/first: the block-table window; cache_k/v: element
    // base of the caches; tok_stride = Hkv*D; head_off = hk*D (elements).
    __device__ __forceinline__ void load(const uint16_t* __restrict__ cache_k,
                                         const uint16_t* __restrict__ cache_v, const int* win,
                                         int first, int j0, int kv_len, int bs_log2,
                                         int tok_stride, int head_off, int tid) {
        const int bs_mask = (1 << bs_log2) - 1;
        const int last = kv_len - 1;
        const int64_t page_stride = (int64_t)tok_stride << bs_log2;
        if (does_k(tid)) {
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int idx = k_index(tid, i);
                const int row = idx / CPR, c = idx % CPR;
                const int tok = min(j0 + row, last);
                const int page = win[(tok >> bs_log2) - first];
                const uint16_t* src = cache_k + page * page_stride +
                                      ((tok & bs_mask) * tok_stride + head_off + c * 8);
                kreg[i] = ld16<STREAM>(src);
            }
        }
        if (does_v(tid)) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int u = tid + i * NT;
                const int quad = u % QPT, dc = u / QPT;
                const int tok0 = min(j0 + swap23(quad * 4), last);   // keys tok0 .. tok0+3
                const int page = win[(tok0 >> bs_log2) - first];
                const uint16_t* src = cache_v + page * page_stride +
                                      ((tok0 & bs_mask) * tok_stride + head_off + dc * 8);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int step = (tok0 + e <= last) ? e : 0;
                    vreg[i][e] = ld16<STREAM>(src + step * tok_stride);
                }
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t* lds, int j0, int kv_len, int tid) const {
        uint8_t* lk = lds;
        uint8_t* lv = lds + K_BYTES;
        const u32x4_t zero = {0u, 0u, 0u, 0u};
        if (does_k(tid)) {
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
                const int idx = k_index(tid, i);
                const int row = idx / CPR, c = idx % CPR;
                const u32x4_t v = (j0 + row < kv_len) ? kreg[i] : zero;
                *reinterpret_cast<u32x4_t*>(lk + row * KP + c * 16) = v;
            }
        }
        if (does_v(tid)) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int u = tid + i * NT;
                const int quad = u % QPT, dc = u / QPT;
                const int tok0 = j0 + swap23(quad * 4);
                u32x4_t rows[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) rows[e] = (tok0 + e < kv_len) ? vreg[i][e] : zero;
                uint8_t* dst = lv + (dc * 8) * VP + quad * 8;   // slots quad*4 .. quad*4+3
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
                    const int w = x >> 1;
                    u32x2_t out;
                    out.x = __builtin_amdgcn_perm(rows[1][w], rows[0][w], sel);
                    out.y = __builtin_amdgcn_perm(rows[3][w], rows[2][w], sel);
                    *reinterpret_cast<u32x2_t*>(dst + x * VP) = out;
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Paged K/V tile loader for an fp8 e4m3 cache (bytes, same page layout).
//
// Fills exactly the LDS tile PagedTile16 fills (16-bit K rows, V^T with key
// slots swap23), converting each e4m3 code to the 16-bit type of the query
// with v_cvt_scalef32_pk_{bf16,f16}_fp8 at scale 1: every e4m3 value is exact
// in bf16 and in f16, so the products see the decoded codes unchanged; the
// per-tensor descales are applied outside (K's to the score scale, V's to O).
// Work per 32-key tile and 64 lanes: K in 16-byte chunks (16 codes), D/32
// per lane; V in units of 4 keys x 16 dims (D/2 units: lanes below that take
// one each), widened and transposed in registers like PagedTile16's 4 x 8
// units.  Keys past kv_len read row kv_len - 1 and are zeroed when stored.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ u32x4_t widen_lo(u32x4_t c) {   // codes 0..7 of 16
    u32x4_t r;
    if constexpr (BF16) {
        r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.f, false));
        r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.f, true));
        r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.f, false));
        r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.f, true));
    } else {
        r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.f, false));
        r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, 1.f, true));
        r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.f, false));
        r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, 1.f, true));
    }
    return r;
}

template <bool BF16>
__device__ __forceinline__ u32x4_t widen_hi(u32x4_t c) {   // codes 8..15 of 16
    return widen_lo<BF16>(u32x4_t{c.z, c.w, 0u, 0u});
}

template <int D, bool BF16>
struct PagedTile8 {
    static constexpr int BN = 32;
    static constexpr int CPR8 = D / 16;               // 16-byte fp8 chunks per key row
    static constexpr int KPL = BN * CPR8 / 64;        // K chunks per lane
    static constexpr int NVU = BN / 4 * CPR8;         // V units (4 keys x 16 dims)
    static_assert(KPL >= 1 && BN * CPR8 % 64 == 0 && NVU <= 64, "tile does not fit one wave");
    static constexpr int KP = k_pitch<D>();
    static constexpr int VP = vt_pitch<BN>();
    static constexpr int K_BYTES = BN * KP;
    static constexpr int V_BYTES = D * VP;
    static constexpr int BYTES = K_BYTES + V_BYTES;

    u32x4_t kreg[KPL];
    u32x4_t vreg[4];

    __device__ __forceinline__ static u32x4_t ld(const uint8_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    }

    // Issue the loads for keys [j0, j0 + 32) of one sequence (kv_len >= 1).
    // win/first: block-table window; tok_stride = Hkv*D, head_off = hk*D
    // (bytes = elements).
    __device__ __forceinline__ void load(const uint8_t* __restrict__ cache_k,
                                         const uint8_t* __restrict__ cache_v, const int* win,
                                         int first, int j0, int kv_len, int bs_log2,
                                         int tok_stride, int head_off, int lane) {
        const int bs_mask = (1 << bs_log2) - 1;
        const int last = kv_len - 1;
        const int64_t page_stride = (int64_t)tok_stride << bs_log2;
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int idx = lane + 64 * i;
            const int row = idx / CPR8, c = idx % CPR8;
            const int tok = min(j0 + row, last);
            const int page = win[(tok >> bs_log2) - first];
            kreg[i] = ld(cache_k + page * page_stride + ((tok & bs_mask) * tok_stride + head_off + c * 16));
        }
        if (NVU == 64 || lane < NVU) {
            const int quad = lane % (BN / 4), dc = lane / (BN / 4);
            const int tok0 = min(j0 + swap23(quad * 4), last);   // keys tok0 .. tok0+3, one page
            const int page = win[(tok0 >> bs_log2) - first];
            const uint8_t* src = cache_v + page * page_stride +
                                 ((tok0 & bs_mask) * tok_stride + head_off + dc * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int step = (tok0 + e <= last) ? e : 0;
                vreg[e] = ld(src + step * tok_stride);
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t* lds, int j0, int kv_len, int lane) const {
        uint8_t* lk = lds;
        uint8_t* lv = lds + K_BYTES;
        const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
            const int idx = lane + 64 * i;
            const int row = idx / CPR8, c = idx % CPR8;
            const bool in = j0 + row < kv_len;
            *reinterpret_cast<u32x4_t*>(lk + row * KP + c * 32) = in ? widen_lo<BF16>(kreg[i]) : zero;
            *reinterpret_cast<u32x4_t*>(lk + row * KP + c * 32 + 16) = in ? widen_hi<BF16>(kreg[i]) : zero;
        }
        if (NVU < 64 && lane >= NVU) return;
        const int quad = lane % (BN / 4), dc = lane / (BN / 4);
        const int tok0 = j0 + swap23(quad * 4);
        uint8_t* dst = lv + (dc * 16) * VP + quad * 8;   // slots quad*4 .. quad*4+3
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            u32x4_t rows[4];   // 4 keys x 8 dims (16-bit) of dims half*8 .. half*8+7
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u32x4_t w = half ? widen_hi<BF16>(vreg[e]) : widen_lo<BF16>(vreg[e]);
                rows[e] = (tok0 + e < kv_len) ? w : zero;
            }
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
                const int w = x >> 1;
                u32x2_t out;
                out.x = __builtin_amdgcn_perm(rows[1][w], rows[0][w], sel);
                out.y = __builtin_amdgcn_perm(rows[3][w], rows[2][w], sel);
                *reinterpret_cast<u32x2_t*>(dst + (half * 8 + x) * VP) = out;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Per-wave attention state for QB blocks of 32 query rows (one row per lane
// column) and the tile step.
//
// Online softmax with a lazily updated running max: m only moves when some
// row's tile max exceeds it by more than kRescaleSlack (log2 units), so the
// O^T rescale -- D/32 x 16 multiplies per row block -- runs on a handful of
// tiles instead of every tile.  Between updates the probabilities
// exp2(s*c - m) may reach 2^kRescaleSlack; the final O/l and LSE are
// unchanged by the choice of m, which cancels exactly.
// ---------------------------------------------------------------------------
constexpr float kRescaleSlack = 8.0f;

template <int D, int QB>
struct RowsState {
    u32x4_t q[QB][D / 16];    // Q^T operand: 8 dims (16t + 8g ..) per lane-half
    f32x16_t o[D / 32][QB];   // O^T accumulators (unnormalised)
    float m[QB];              // running max of score * scale * log2(e) (may lag)
    float l[QB];              // running sum of exp2(score * c - m)
    int lo[QB], hi[QB];       // visible key interval [lo, hi) of the lane's row

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m[qb] = kNegInf;
            l[qb] = 0.f;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db][qb] = f32x16_t{};
        }
    }
};

// Flip the sign of every 16-bit element of a Q operand (a negative scale is
// applied as |scale| on -q, which keeps the running max a max).
__device__ __forceinline__ u32x4_t neg16x8(u32x4_t v) {
    const uint32_t s = 0x80008000u;
    return u32x4_t{v.x ^ s, v.y ^ s, v.z ^ s, v.w ^ s};
}

// One key tile against the wave's rows, reading K and Vt from LDS.  The LDS
// tile is BN keys wide (starting at key j0); this wave processes the NKB
// 32-key blocks kb0 .. kb0+NKB-1 of it.  c = |scale| * log2(e) >= 0.  MASKED
// evaluates each row's visible interval [lo, hi); otherwise every key of the
// processed blocks is visible to every row.
template <int D, int BN, int NKB, int QB, bool BF16, bool MASKED, bool CAP = false>
__device__ __forceinline__ void tile_step(RowsState<D, QB>& st, const uint8_t* lds, int j0,
                                          int kb0, float c, float cap_in2 = 0.f,
                                          float cap_out = 0.f) {
    constexpr int KP = k_pitch<D>();
    constexpr int VP = vt_pitch<BN>();
    const int lane = lane_id();
    const int col = lane & 31, g = lane >> 5;
    const uint8_t* lk = lds + col * KP + g * 16;                 // + row block, + 32 t
    const uint8_t* lv = lds + BN * KP + col * VP + g * 16;       // + 32 VP db, + 16 chunk

    f32x16_t s[NKB][QB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16_t{};

#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                lk + (kb0 + kb) * 32 * KP + t * 32);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32<BF16>(a, st.q[qb][t], s[kb][qb]);
        }
    }

    // mask (select) and raw row max
    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (MASKED) {
                    const int key = j0 + (kb0 + kb) * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (!(key >= st.lo[qb] && key < st.hi[qb])) s[kb][qb][r] = kNegInf;
                }
                // capped scores are already in log2 units (c = 1 below)
                if constexpr (CAP) s[kb][qb][r] = cap_score(s[kb][qb][r], cap_in2, cap_out);
                mx[qb] = fmaxf(mx[qb], s[kb][qb][r]);
            }

    if constexpr (CAP) c = 1.f;
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mx[qb] = pair_max(mx[qb]);
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
            for (int db = 0; db < D / 32; ++db) st.o[db][qb] *= alpha;
        }
    }

    // probabilities, row sums, packed P^T operands
    float rs[QB];
    u32x4_t pb[NKB][2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        rs[qb] = 0.f;
        const float nm = (st.m[qb] == kNegInf) ? 0.f : -st.m[qb];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // masked scores are -inf; with c == 0 the product would be NaN
                p[r] = fast_exp2(__builtin_fmaf(s[kb][qb][r], c, nm));
                if constexpr (MASKED) p[r] = (s[kb][qb][r] == kNegInf) ? 0.f : p[r];
                rs[qb] += p[r];
            }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                u32x4_t w;
                w.x = pack2<BF16>(p[8 * tp + 0], p[8 * tp + 1]);
                w.y = pack2<BF16>(p[8 * tp + 2], p[8 * tp + 3]);
                w.z = pack2<BF16>(p[8 * tp + 4], p[8 * tp + 5]);
                w.w = pack2<BF16>(p[8 * tp + 6], p[8 * tp + 7]);
                pb[kb][tp][qb] = w;
            }
        }
        st.l[qb] += pair_sum(rs[qb]);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                    lv + db * 32 * VP + (4 * (kb0 + kb) + 2 * tp) * 16);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    st.o[db][qb] = mfma32<BF16>(a, pb[kb][tp][qb], st.o[db][qb]);
            }
}

// Bytes of LDS one wave needs for store_rows_lds: 32 rows of D 16-bit
// values, each row padded by 16 bytes so the lanes' 8-byte writes of one
// register group spread over all banks.
template <int D>
constexpr int kStoreRowPitch = 2 * D + 16;
template <int D>
constexpr int kStoreSliceBytes = 32 * kStoreRowPitch<D>;

// Write the normalised O (O^T accumulators / l, 0 when l == 0) of a wave's
// 32 query rows to their token-major output rows, through LDS: each lane
// first puts its half row (the accumulator rows it holds) into `slice` (row
// = its column), then the wave stores whole rows, 16 contiguous bytes per
// lane, so one store instruction covers 64 / (D / 8) complete rows instead
// of 16 bytes in each of 32 rows.  row_ptr(rr) gives the output row of local row
// rr (0..31), or null for a row that is not stored.  `slice` must be this
// wave's alone; the wave's LDS operations complete in order, so its reads
// see its writes without a barrier.
template <int D, bool BF16, class RowPtr>
__device__ __forceinline__ void store_rows_lds(const f32x16_t* o_db, float l, uint8_t* slice,
                                               const RowPtr& row_ptr) {
    constexpr int PITCH = kStoreRowPitch<D>;
    constexpr int CPR = D / 8;      // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;   // rows per store instruction
    const int lane = lane_id();
    const int col = lane & 31, g = lane >> 5;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d = db * 32 + 8 * rq + 4 * g;
            u32x2_t w;
            w.x = pack2<BF16>(o_db[db][4 * rq + 0] * inv, o_db[db][4 * rq + 1] * inv);
            w.y = pack2<BF16>(o_db[db][4 * rq + 2] * inv, o_db[db][4 * rq + 3] * inv);
            *reinterpret_cast<u32x2_t*>(slice + col * PITCH + 2 * d) = w;
        }
    const int ch = lane % CPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int rr = i * RPI + lane / CPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(slice + rr * PITCH + 16 * ch);
        uint16_t* dst = row_ptr(rr);
        if (dst != nullptr) *reinterpret_cast<u32x4_t*>(dst + 8 * ch) = v;
    }
}

}  // namespace attn
