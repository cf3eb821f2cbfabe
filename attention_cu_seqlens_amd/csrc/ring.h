// Multi-stage LDS ring for paged K/V tiles of 16-bit dtypes, filled with
// direct global->LDS loads (no register staging), plus the MFMA tile
// products that read it.
//
// Tile layout in LDS (both K and V): row-major, one row per key, D/8
// 16-byte chunks per row; logical chunk c of row r is stored at chunk
// c ^ swz<D>(r).  gfx950's LDS serves 256 bytes per clock (64 banks = 16
// groups of 16 bytes), so the swizzle makes
//   * the 16 lanes that read one chunk of 16 consecutive K rows (the A
//     operand of S^T = K.Q^T, 16 bytes per lane) hit 16 bank groups;
//   * the 32 lanes of one transposed V read (4 rows x 4 chunks x 2 halves,
//     8 bytes per lane) hit all 64 banks once.
// A direct LDS load writes 64 lanes x 16 bytes = 1 KB of consecutive LDS per
// instruction, so each lane simply fetches the global chunk that belongs at
// its LDS position.
//
// V is consumed with the gfx950 transposed LDS read (16-bit elements, 8 bytes
// per lane): within each group of 16 lanes, output lane i receives element
// i%4 of the 8-byte rows read by lanes 4e + i/4, e = 0..3.  Pointing lane
// 4e + q of the group at V[key0 + e][d0 + 4q .. +3] gives lane i the four keys
// key0..key0+3 of dimension d0 + i -- the key-contiguous V^T operand, read
// from a plain row-major V tile (the layout question of the FlexAttention fp8
// commit, "[FlexAttention] Enforce Q,K,V memory layouts for fp8 flex
// attention...", Context, answered in the LDS read instead of in HBM).
#pragma once

#include "device_common.h"

namespace attn {

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (other counters untouched).
__host__ __device__ constexpr unsigned vmcnt_imm(int n) {
    return 0x0F70u | (unsigned)(n & 15) | ((unsigned)((n >> 4) & 3) << 14);
}

// Workgroup barrier without a memory fence: the direct-to-LDS loads of later
// tiles stay in flight across it (each wave waits for its own loads with an
// explicit vmcnt first).  The memory clobber keeps the compiler from moving
// LDS accesses across it.
// Every LDS read this wave issued has returned before it signals the barrier
// (lgkmcnt(0)), so a stage may be refilled right after the barrier.
__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07Fu);   // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// D = 128: 256-byte rows, one row spans all banks; the low two row bits pick
// the 4-chunk group of a V read and bits 2-3 separate the 16 K rows.
// D = 64: 128-byte rows, row parity already selects the bank half.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// One direct global->LDS load of 16 bytes per lane: lane i's bytes land at
// LDS byte address lds + 16*i (lds must be wave-uniform; lds_addr() gives the
// address of a __shared__ object).  Written as
// inline asm so the compiler does not drain it with vmcnt(0) before every
// later LDS read (it cannot tell ring stages apart); the code that reads a
// stage waits with an explicit vmcnt first.  The instruction has no
// destination register.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)(p);
}

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m0), "v"(gptr)
                 : "memory", "m0");
}

// The 4-byte form: lane i's 4 bytes land at LDS byte address lds + 4*i.
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(m0), "v"(gptr)
                 : "memory", "m0");
}

// The same load with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset: no per-lane address arithmetic.
// The base goes through readfirstlane so it is in SGPRs even where the
// compiler cannot prove it uniform (a no-op where it can).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    const uint64_t a = (uint64_t)(uintptr_t)sbase;
    // readfirstlane returns int: take each half back to uint32_t before
    // widening so the low half is not sign-extended into the high one.
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t u = ((uint64_t)hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(u)
                 : "memory", "m0");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ u32x2_t ds_read_tr16(const uint8_t* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// Ring of K/V tiles filled by NL loading waves.  Loading wave wl fetches the
// RW consecutive key rows [wl*RW, (wl+1)*RW) of a tile; tiles start on
// multiples of 16 and pages hold at least 16 keys, so those rows lie in one
// page: one page id per wave and tile, and a wave-uniform source address.
template <int D, int BN, int NL>
struct Ring16 {
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static constexpr int ROWB = D * 2;          // bytes per row
    static constexpr int TILE = BN * ROWB;      // bytes of one K (or V) tile
    static constexpr int STAGE = 2 * TILE;      // K tile then V tile
    static constexpr int RPI = 64 / CPR;        // rows per 1 KB load instruction
    static constexpr int IPW = TILE / 1024 / NL;  // load instructions per wave per tensor
    static_assert(TILE % (1024 * NL) == 0, "tile does not divide over the waves");
    static constexpr int RW = IPW * RPI;
    static_assert(RW == 16, "a loading wave's rows must be one aligned 16-key group");

    // Load instruction i of loading wave wl puts lane l's 16 bytes at tile
    // row row(i) = (wl*IPW + i)*RPI + l/CPR, logical chunk chunk(i) (the
    // swizzle applied); voff[i] is that chunk's byte offset from the wave's
    // first row in the cache.
    uint32_t voff[IPW];

    __device__ __forceinline__ static int row(int lane, int wl, int i) {
        return (wl * IPW + i) * RPI + lane / CPR;
    }
    __device__ __forceinline__ static int chunk(int lane, int wl, int i) {
        return (lane % CPR) ^ swz<D>(row(lane, wl, i));
    }

    __device__ __forceinline__ void init(int lane, int wl, int tok_stride) {
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            voff[i] = (uint32_t)(((row(lane, wl, i) - wl * RW) * tok_stride +
                                  chunk(lane, wl, i) * 8) * 2);
    }

    // Window slot of the page holding this wave's rows of the tile at j0.
    __device__ __forceinline__ static int slot(int j0, int first, int bs_log2, int wl) {
        return ((j0 + wl * RW) >> bs_log2) - first;
    }

    // True when all of this wave's rows of the tile at j0 are below kv_len.
    __device__ __forceinline__ static bool whole(int j0, int kv_len, int wl) {
        return j0 + (wl + 1) * RW <= kv_len;
    }

    struct Src {
        const uint16_t* k;
        const uint16_t* v;
    };

    // Wave-uniform source rows of a whole() tile; page = win[slot()].
    __device__ __forceinline__ static Src src(const uint16_t* cache_k, const uint16_t* cache_v,
                                              int page, int j0, int wl, int bs_log2,
                                              int tok_stride, int head_off) {
        const int r0 = __builtin_amdgcn_readfirstlane(j0 + wl * RW);
        const int pg = __builtin_amdgcn_readfirstlane(page);
        const int64_t off = ((int64_t)pg * tok_stride << bs_log2) +
                            (((r0 & ((1 << bs_log2) - 1)) * tok_stride) + head_off);
        return Src{cache_k + off, cache_v + off};
    }

    // Load i (< IPW) of this wave's K rows (v false) or V rows (v true) of a
    // whole() tile.
    __device__ __forceinline__ void dma_half(int i, bool v, const Src& sr, uint32_t stage,
                                             int wl) const {
        dma16_s(v ? sr.v : sr.k, voff[i], stage + (v ? TILE : 0) + (wl * IPW + i) * 1024);
    }

    // This wave's K rows (v false) or V rows (v true) of the tile at j0 at
    // once (kv_len >= 1).  Rows past kv_len read row kv_len - 1: they hold
    // finite values and every key past kv_len is masked to probability 0 by
    // the caller.  `page` is win[slot()], read by the caller ahead of time
    // (any value when the tile is not whole()).
    __device__ __forceinline__ void issue_half(bool v, uint32_t stage, const uint16_t* cache_k,
                                               const uint16_t* cache_v, const int* win, int first,
                                               int j0, int kv_len, int bs_log2, int tok_stride,
                                               int head_off, int wl, int page) const {
        if (whole(j0, kv_len, wl)) {
            const Src sr = src(cache_k, cache_v, page, j0, wl, bs_log2, tok_stride, head_off);
#pragma unroll
            for (int i = 0; i < IPW; ++i) dma_half(i, v, sr, stage, wl);
            return;
        }
        const int bs_mask = (1 << bs_log2) - 1;
        const int64_t page_stride = (int64_t)tok_stride << bs_log2;
        const int lane = lane_id();
        const uint16_t* base = v ? cache_v : cache_k;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int tok = min(j0 + row(lane, wl, i), kv_len - 1);
            const int pg = win[(tok >> bs_log2) - first];
            const int64_t off = pg * page_stride +
                                ((tok & bs_mask) * tok_stride + head_off + chunk(lane, wl, i) * 8);
            dma16(base + off, stage + (v ? TILE : 0) + (wl * IPW + i) * 1024);
        }
    }
};

// Callback run after each MFMA of a tile product (step = MFMA index within
// the product) when the caller has nothing to interleave.
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

// Operand prefetch depth of the MFMA stream, in MFMA steps: the LDS reads of
// step t + PD issue before the MFMA of step t, so LDS latency hides under the
// MFMAs; sched_barrier pins that order against the scheduler.
#ifndef ATTN_STREAM_PREFETCH
#define ATTN_STREAM_PREFETCH 6
#endif
constexpr int kStreamPrefetch = ATTN_STREAM_PREFETCH;

// Lane offsets of the transposed V reads of the P.V product: within each
// group of 16 lanes, lane j reads row r0 + 16*tp + 32*kb (and the row 8
// below) at chunk c0 + 4*db.  Rows r0 + 16*tp + 32*kb keep the swizzle of r0
// (it depends on the row mod 16), row r0 + 8 has its own.  These are the
// offsets of db = 0 for both rows; db adds (4*db << 4) by XOR (those chunk
// bits of c0 are zero).
template <int D>
__device__ __forceinline__ void pv_offsets(uint32_t& lo0, uint32_t& hi0) {
    constexpr int ROWB = D * 2;
    const int lane = lane_id();
    const int j = lane & 15, h = lane >> 4, gv = h >> 1;
    const int r0 = 4 * gv + (j >> 2);
    const int c0 = (16 * (h & 1) + 4 * (j & 3)) >> 3;
    lo0 = (uint32_t)(r0 * ROWB + (j & 1) * 8 + ((c0 ^ swz<D>(r0)) << 4));
    hi0 = (uint32_t)((r0 + 8) * ROWB + (j & 1) * 8 + ((c0 ^ swz<D>(r0 + 8)) << 4));
}

// V^T operand of P.V step i (db, kb, tp) read from the V tile at vt.
template <int D, int BN>
__device__ __forceinline__ u32x4_t pv_frag(const uint8_t* vt, uint32_t lo0, uint32_t hi0, int i) {
    constexpr int ROWB = D * 2;
    constexpr int NKB = BN / 32;
    const int db = i / (NKB * 2), kb = (i / 2) % NKB, tp = i % 2;
    const uint8_t* p0 = vt + (kb * 32 + 16 * tp) * ROWB;
    const uint32_t x = (uint32_t)(db << 6);
    const u32x2_t l2 = ds_read_tr16(p0 + (lo0 ^ x));
    const u32x2_t h2 = ds_read_tr16(p0 + (hi0 ^ x));
    return u32x4_t{l2.x, l2.y, h2.x, h2.y};
}

// The MFMA work of one pipeline phase as a single stream, so the operand
// prefetch runs on across the boundary between the two products instead of
// refilling at the start of each:
//   PV: O^T[db] += V_tile^T(db) . P^T, P^T packed per (key block, 16-key
//       step): (D/32) * (BN/32) * 2 MFMAs (steps db, kb, tp; `hook` after
//       each);
//   QK: S^T[kb] = K_tile(kb) . Q^T for the BN/32 key blocks: (D/16) * (BN/32)
//       MFMAs (steps t, kb).
template <int D, int BN, bool BF16, bool PV, bool QK, class Hook>
__device__ __forceinline__ void mfma_stream16(f32x16_t (&o)[D / 32], f32x16_t (&s)[BN / 32],
                                              const u32x4_t (&pb)[BN / 32][2],
                                              const u32x4_t (&q)[D / 16], const uint8_t* vt,
                                              const uint8_t* kt, const Hook& hook) {
    static_assert(PV || QK, "empty stream");
    constexpr int ROWB = D * 2;
    constexpr int NKB = BN / 32;
    constexpr int NPV = PV ? (D / 32) * NKB * 2 : 0;
    constexpr int N = NPV + (QK ? (D / 16) * NKB : 0);
    constexpr int PD = kStreamPrefetch < N ? kStreamPrefetch : N;
    uint32_t lo0, hi0;
    pv_offsets<D>(lo0, hi0);
    // K: lane offset of chunk g of row col (rows kb*32 + col share their low
    // 5 bits, so one swizzle serves every key block).  Step t reads chunk
    // 2t + g: this offset XOR (2t << 4); row bits sit above bit 7.
    const int lane = lane_id();
    const int col = lane & 31, g = lane >> 5;
    uint32_t lok = (uint32_t)(col * ROWB + ((g ^ swz<D>(col)) << 4));
    // The empty asm keeps the compiler from hoisting the XORed offsets of
    // every step out of the tile loop into registers held across it.
    asm volatile("" : "+v"(lo0), "+v"(hi0), "+v"(lok));
    auto frag = [&](int i) {
        if (i < NPV) return pv_frag<D, BN>(vt, lo0, hi0, i);
        const int k = i - NPV, t = k / NKB, kb = k % NKB;
        return *reinterpret_cast<const u32x4_t*>(kt + kb * 32 * ROWB + (lok ^ (uint32_t)(t << 5)));
    };
    u32x4_t a[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) a[i] = frag(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        // buffer slot of step k: k % (PD + 1)
        if (i + PD < N) a[(i + PD) % (PD + 1)] = frag(i + PD);
        __builtin_amdgcn_sched_barrier(0);
        const u32x4_t op = a[i % (PD + 1)];
        if (i < NPV) {
            const int db = i / (NKB * 2), kb = (i / 2) % NKB, tp = i % 2;
            o[db] = mfma32<BF16>(op, pb[kb][tp], o[db]);
            hook(i);
        } else {
            const int k = i - NPV, t = k / NKB, kb = k % NKB;
            s[kb] = mfma32<BF16>(op, q[t], t == 0 ? f32x16_t{} : s[kb]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Online softmax of one tile's scores for one 32-row block (QB = 1).
// s: raw S^T accumulators (masked entries already -inf); c > 0, so a masked
// score gives exp2(-inf) = 0 with no further test (a zero scale is passed
// as a tiny positive c, which leaves every visible weight exactly 1);
// on return pb holds the packed probabilities, m may have moved (then *need
// is set and alpha holds exp2(m_old - m_new)), and lpart accumulated this
// lane's partial row sum (relative to the final m after any rescale).  CAP
// first replaces every score by its capped value in log2 units (cap_score),
// after which the scale factor is 1.
template <int BN, bool BF16, bool CAP = false>
__device__ __forceinline__ void softmax_tile(f32x16_t (&s)[BN / 32], float c, float& m,
                                             float& lpart, u32x4_t (&pb)[BN / 32][2],
                                             float& alpha, bool& need, float cap_in2 = 0.f,
                                             float cap_out = 0.f) {
    if constexpr (CAP) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = cap_score(s[kb][r], cap_in2, cap_out);
        c = 1.f;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);
    mx = (mx == kNegInf) ? kNegInf : mx * c;
    // Each row moves its own running max (only the rescale branch is
    // wave-uniform), so a row's arithmetic does not depend on which rows
    // share its wave: a query head gives the same bits whether or not it is
    // packed with the other heads of its GQA group.
    const bool up = mx > m + kRescaleSlack;
    need = __any(up);
    const float mnew = up ? mx : m;
    alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m - mnew);
    m = mnew;
    const float nm = (mnew == kNegInf) ? 0.f : -mnew;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = fast_exp2(__builtin_fmaf(s[kb][r], c, nm));
            rs += p[r];
        }
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            u32x4_t wv;
            wv.x = pack2<BF16>(p[8 * tp + 0], p[8 * tp + 1]);
            wv.y = pack2<BF16>(p[8 * tp + 2], p[8 * tp + 3]);
            wv.z = pack2<BF16>(p[8 * tp + 4], p[8 * tp + 5]);
            wv.w = pack2<BF16>(p[8 * tp + 6], p[8 * tp + 7]);
            pb[kb][tp] = wv;
        }
    }
    lpart = lpart * alpha + rs;
}

}  // namespace attn
