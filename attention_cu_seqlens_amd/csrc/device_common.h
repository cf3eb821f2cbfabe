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

// Exchange with lane ^ 32 (the other half of a 32-wide MFMA column).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = min(x, __shfl_xor(x, s, 64));
    return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = max(x, __shfl_xor(x, s, 64));
    return x;
}

// Bits 2 and 3 of a key index swapped.  The accumulator rows a lane feeds to
// one 16-key P^T step are keys {4g..4g+3} and {8+4g..8+4g+3}; storing key k at
// V^T slot swap23(k) makes those 8 keys one contiguous 16-byte LDS read.
__device__ __forceinline__ int swap23(int k) {
    return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// 16-byte chunk swizzles for the LDS tiles (bank-conflict avoidance).
__device__ __forceinline__ int k_swz(int row) { return row & 7; }
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

// ---------------------------------------------------------------------------
// Paged K/V tile loader for 16-bit dtypes.
//
// A tile is BN consecutive keys of one sequence and one kv head.  LDS gets
//   K  [BN][D]   16-bit, row = key, 16-byte chunk c stored at c ^ k_swz(row)
//   Vt [D][BN]   16-bit, row = dim, key k at slot swap23(k); 16-byte chunk c
//                stored at c ^ vt_swz(d)
// Keys at or past kv_len are zero-filled (the cache may hold NaN there).
// Each thread owns KPT 16-byte K chunks and VPT V units of 4 keys x 8 dims;
// a V unit is transposed in registers (4 rows x 4 dwords -> 8 dim rows x 2
// dwords) and written as eight 8-byte LDS stores.
// ---------------------------------------------------------------------------
template <int D, int BN, int NT>
struct PagedTile16 {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per key row
    static constexpr int NV = (BN / 4) * CPR;         // V units per tile
    static constexpr int VPT = NV / NT;
    static constexpr int KPT = BN * CPR / NT;
    static_assert(VPT >= 1 && NV % NT == 0, "V units must divide evenly");
    static_assert(KPT >= 1 && (BN * CPR) % NT == 0, "K chunks must divide evenly");
    static constexpr int K_BYTES = BN * D * 2;
    static constexpr int V_BYTES = D * BN * 2;
    static constexpr int BYTES = K_BYTES + V_BYTES;

    u32x4_t kreg[KPT];
    u32x4_t vreg[VPT][4];

    // Issue the global loads for keys [j0, j0 + BN) of one sequence.
    //   cache_k/v: element base of the caches; table: this sequence's
    //   block_table row; tok_stride = Hkv*D; head_off = hk*D (elements).
    __device__ __forceinline__ void load(const uint16_t* __restrict__ cache_k,
                                         const uint16_t* __restrict__ cache_v,
                                         const int32_t* __restrict__ table, int j0, int kv_len,
                                         int bs_log2, int tok_stride, int head_off, int tid) {
        const int bs_mask = (1 << bs_log2) - 1;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / CPR, c = idx % CPR;
            const int tok = j0 + row;
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (tok < kv_len) {
                const int64_t page = table[tok >> bs_log2];
                const int64_t off = ((page << bs_log2) + (tok & bs_mask)) * tok_stride + head_off +
                                    c * 8;
                v = *reinterpret_cast<const u32x4_t*>(cache_k + off);
            }
            kreg[i] = v;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int u = tid + i * NT;
            const int dc = u % CPR, quad = u / CPR;
            const int key0 = swap23(quad * 4);           // 4 consecutive keys key0..key0+3
            const int tok0 = j0 + key0;
            int64_t base = 0;
            if (tok0 < kv_len) {
                const int64_t page = table[tok0 >> bs_log2];
                base = ((page << bs_log2) + (tok0 & bs_mask)) * tok_stride + head_off + dc * 8;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (tok0 + e < kv_len)
                    v = *reinterpret_cast<const u32x4_t*>(cache_v + base + (int64_t)e * tok_stride);
                vreg[i][e] = v;
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
        uint8_t* lk = lds;
        uint8_t* lv = lds + K_BYTES;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            const int row = idx / CPR, c = idx % CPR;
            *reinterpret_cast<u32x4_t*>(lk + row * (D * 2) + ((c ^ k_swz(row)) << 4)) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int u = tid + i * NT;
            const int dc = u % CPR, quad = u / CPR;
            const int chunk = quad >> 1, half = quad & 1;   // slots quad*4 .. quad*4+3
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int d = dc * 8 + x;
                const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
                const int w = x >> 1;
                u32x2_t out;
                out.x = __builtin_amdgcn_perm(vreg[i][1][w], vreg[i][0][w], sel);
                out.y = __builtin_amdgcn_perm(vreg[i][3][w], vreg[i][2][w], sel);
                *reinterpret_cast<u32x2_t*>(lv + d * (BN * 2) + ((chunk ^ vt_swz(d)) << 4) +
                                            half * 8) = out;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Per-wave attention state for QB blocks of 32 query rows (one row per lane
// column) and the tile step.
// ---------------------------------------------------------------------------
template <int D, int QB>
struct RowsState {
    u32x4_t q[QB][D / 16];    // Q^T operand: 8 dims (16t + 8g ..) per lane-half
    f32x16_t o[D / 32][QB];   // O^T accumulators (unnormalised)
    float m[QB];              // running max of scores * scale * log2(e)
    float l[QB];              // running sum of exp2(score - m)
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

// One key tile against the wave's rows, reading K and Vt from LDS.  The LDS
// tile is BN keys wide (starting at key j0); this wave processes the NKB
// 32-key blocks kb0 .. kb0+NKB-1 of it.  c = scale * log2(e).  MASKED
// evaluates each row's visible interval [lo, hi); otherwise every key of the
// processed blocks is visible to every row.
template <int D, int BN, int NKB, int QB, bool BF16, bool MASKED>
__device__ __forceinline__ void tile_step(RowsState<D, QB>& st, const uint8_t* lds, int j0,
                                          int kb0, float c) {
    const uint8_t* lk = lds;
    const uint8_t* lv = lds + BN * D * 2;
    const int lane = lane_id();
    const int col = lane & 31, g = lane >> 5;

    f32x16_t s[NKB][QB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16_t{};

#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int row = (kb0 + kb) * 32 + col;
            const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                lk + row * (D * 2) + (((2 * t + g) ^ k_swz(row)) << 4));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32<BF16>(a, st.q[qb][t], s[kb][qb]);
        }
    }

    // scale, mask, row max
    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[kb][qb][r] * c;
                if constexpr (MASKED) {
                    const int key = j0 + (kb0 + kb) * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    x = (key >= st.lo[qb] && key < st.hi[qb]) ? x : kNegInf;
                }
                s[kb][qb][r] = x;
                mx[qb] = fmaxf(mx[qb], x);
            }

    float alpha[QB], msub[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mx[qb] = fmaxf(mx[qb], xor32(mx[qb]));
        const float mnew = fmaxf(st.m[qb], mx[qb]);
        msub[qb] = (mnew == kNegInf) ? 0.f : mnew;
        alpha[qb] = fast_exp2(st.m[qb] - msub[qb]);
        st.m[qb] = mnew;
    }

    // probabilities, row sums, packed P^T operands
    float rs[QB];
    u32x4_t pb[NKB][2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) rs[qb] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = fast_exp2(s[kb][qb][r] - msub[qb]);
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

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        rs[qb] += xor32(rs[qb]);
        st.l[qb] = st.l[qb] * alpha[qb] + rs[qb];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) st.o[db][qb] *= alpha[qb];
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int d = db * 32 + col;
                const int chunk = 4 * (kb0 + kb) + 2 * tp + g;
                const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                    lv + d * (BN * 2) + ((chunk ^ vt_swz(d)) << 4));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    st.o[db][qb] = mfma32<BF16>(a, pb[kb][tp][qb], st.o[db][qb]);
            }
}

// Write the normalised O^T of one 32-row block to a token-major output row
// (`orow` points at the row's first element) and return 1/l (0 if l == 0).
template <int D, bool BF16>
__device__ __forceinline__ void store_row(const f32x16_t* o_db, float l, uint16_t* orow) {
    const int g = lane_id() >> 5;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d = db * 32 + 8 * rq + 4 * g;
            u32x2_t w;
            w.x = pack2<BF16>(o_db[db][4 * rq + 0] * inv, o_db[db][4 * rq + 1] * inv);
            w.y = pack2<BF16>(o_db[db][4 * rq + 2] * inv, o_db[db][4 * rq + 3] * inv);
            *reinterpret_cast<u32x2_t*>(orow + d) = w;
        }
}

}  // namespace attn
