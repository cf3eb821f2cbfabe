// Dense varlen fp8 e4m3 attention with a column-major V on gfx950.
//
// The fp8 path of the pytorch commit "[FlexAttention] Enforce Q,K,V memory
// layouts for fp8 flex attention to avoid perf degradation": Q and K are
// row-major, V is column-major ([Hkv, D, total_kv], key-contiguous), which is
// the layout the P.V product wants for its V operand (commit message,
// Context; _enforce_mem_layouts).  Here a V tile is 128 rows (one per
// dimension) of 128 consecutive key bytes, copied straight into LDS.
//
// Both products use the 32x32x64 fp8 MFMA (format E4M3 for both operands,
// no block scale).  S^T = K.Q^T as in the 16-bit kernels; for P^T.V the
// scores of two 32-key blocks form one 64-key operand.  A lane's 32 score
// registers of those blocks are rows {8b + 4g + e} of each block; the K tile
// rows are read through a permutation so that those 32 registers hold keys
// 32g .. 32g+31 of the 64-key group, which makes each lane's V^T operand 32
// consecutive bytes of one V^T row.
//
// Pipeline: the same as the 16-bit prefill kernel -- a four-stage LDS ring
// of K/V^T tiles filled by direct global->LDS loads from the first group of
// four waves, and two groups of waves half a tile apart so that on every SIMD
// one wave issues MFMAs while the other computes a softmax.
//
// Numerics: scores = (scale * dq * dk) * (q8 . k8) in fp32; online softmax in
// fp32; P is rounded to e4m3 (nearest even) for the P.V product and the row
// normaliser l is the sum of those rounded values, so O = dv * (P8 . V8) / l
// is a convex combination of V rows.  The sum is one more MFMA per 64-key
// group with an all-ones operand: every partial sum of at most 64 e4m3
// values in [2^-9, 2^8] is exact in fp32, so this equals the plain sum.
//
// A weight rounded to e4m3 is off by up to 2^-4 of itself.  Over the many
// keys of a fully visible tile these errors average out, but a row whose
// visible keys are few (the first rows of a causal sequence or of a document,
// a narrow window) sees them all in masked tiles.  There P is carried as two
// e4m3 terms, P8 = e4m3(P) and e4m3(P - P8), both multiplied with the same V
// operand and both summed into l: the weight error drops to about 2^-8 of
// the weight, as with 16-bit probabilities, for twice the P.V MFMAs on
// those tiles only.

#include "device_common.h"
#include "kernels.h"
#include "ring.h"

namespace attn {

namespace {

__device__ __forceinline__ f32x16_t mfma_fp8(const i32x8_t& a, const i32x8_t& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

constexpr int D8 = 128;     // head size (bytes per row)
constexpr int BN8 = 128;    // keys per tile
constexpr int kStages8 = 4;

// LDS tile layouts (128-byte rows, 8 chunks of 16 bytes).  gfx950's LDS
// serves 16 lanes x 16 bytes per clock from 64 banks; a row covers half of
// them, so a 16-lane read is conflict-free when its lanes' (row parity,
// stored chunk) pairs are all distinct.
//   K: chunk c of key row r is stored at c ^ kswz(r).  The 16 lanes of one
//      A-operand read take rows that differ in bits 0, 1, 2 (or 3) and 5.
//   V^T: chunk c of dimension row d is stored at c ^ vswz(d); one read takes
//      16 consecutive rows.
__device__ __forceinline__ int kswz(int r) {
    return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 5) & 1) << 2);
}
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

// Key row (within the tile) read by A-operand row j of 32-key block kb.
__device__ __forceinline__ int fp8_krow(int kb, int j) {
    return 64 * (kb >> 1) + 16 * (kb & 1) + 32 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3);
}

// Ring of K / V^T tiles of the fp8 kernel, loaded by four waves.  Loading
// wave wl owns K rows and V^T rows [32 wl, 32 wl + 32) of every tile: four
// direct loads of 1 KB (8 rows) each per tensor.
struct Ring8 {
    static constexpr int TILE = BN8 * D8;          // 16 KB per tensor
    static constexpr int STAGE = 2 * TILE;         // K tile then V^T tile
    static constexpr int IPW = 4;                  // loads per wave per tensor
    static constexpr int LOADS_PER_TILE = 2 * IPW;

    // Lane byte offsets from the wave's first K row and V^T row.  The K
    // swizzle of the lane's row does not change between the wave's loads
    // (rows 32 wl + 8 i + lane / 8 share bits 1, 2 and 5), and the V^T one
    // depends on i only through i & 1, so load i adds a wave-uniform row
    // offset (8 i K rows, 16 (i >> 1) V^T rows) to the scalar base instead of
    // holding one register per load.
    uint32_t koff;
    uint32_t voff[2];
    int k_stride, total_kv;

    __device__ __forceinline__ static int row(int lane, int wl, int i) {
        return 32 * wl + 8 * i + (lane >> 3);
    }
    __device__ __forceinline__ static int kchunk(int lane, int wl, int i) {
        return (lane & 7) ^ kswz(row(lane, wl, i));
    }
    __device__ __forceinline__ static int vchunk(int lane, int wl, int i) {
        return (lane & 7) ^ vswz(row(lane, wl, i));
    }

    __device__ __forceinline__ void init(int lane, int wl, int k_stride_, int total_kv_) {
        k_stride = k_stride_;
        total_kv = total_kv_;
        const int rr = lane >> 3;
        koff = (uint32_t)(rr * k_stride + kchunk(lane, wl, 0) * 16);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            voff[i] = (uint32_t)(8 * i + rr) * (uint32_t)total_kv +
                      (uint32_t)(vchunk(lane, wl, i) * 16);
    }

    struct Src {
        const uint8_t* k;   // K row 32 wl of the tile
        const uint8_t* v;   // V^T row 32 wl, key j0 of the tile
    };

    // Load k (< LOADS_PER_TILE: K first, then V^T) of a tile fetched with
    // wave-uniform bases.  stage: LDS byte address of the ring stage.
    __device__ __forceinline__ void dma(int k, const Src& sr, uint32_t stage, int wl) const {
        const int i = k % IPW;
        if (k < IPW)
            dma16_s(sr.k + (int64_t)(8 * i) * k_stride, koff, stage + (wl * IPW + i) * 1024);
        else
            dma16_s(sr.v + (int64_t)(16 * (i >> 1)) * total_kv, voff[i & 1],
                    stage + TILE + (wl * IPW + i) * 1024);
    }
};

// Per-wave pipeline state of one 32-row block.
struct Fp8Wave {
    f32x16_t s[4];       // scores of the tile waiting for its softmax
    i32x8_t pb[2];       // e4m3 probabilities of the tile waiting for its P.V
    i32x8_t plo[2];      // e4m3 remainders P - pb (masked tiles only)
    f32x16_t o[4];       // O^T accumulators (P8 . V8, unscaled)
    f32x16_t l;          // row sums of P8 (every row of a column holds it)
    float m, alpha;
    bool need;
    bool split;          // the tile waiting for its P.V carries plo
};

// Online softmax of one tile (VALU): mask when partial, cap the scores with
// CAP (in log2 units, scale factor 1 after that), new running max (lazy:
// moved only when some row's tile max exceeds it by more than
// kRescaleSlack), probabilities rounded to e4m3 into pb; a masked tile also
// gets the e4m3 remainders P - pb into plo.
template <bool MASKED, bool CAP>
__device__ __forceinline__ void softmax8(Fp8Wave& st, float c, int j0, int lo, int hi,
                                         float cap_in2, float cap_out) {
    const int g = lane_id() >> 5;
    if constexpr (MASKED) {
        // key k held by register r of block kb is visible iff the unsigned
        // k - lo is below hi - lo (hi >= lo)
        const uint32_t off = (uint32_t)(j0 + 32 * g - lo);
        const uint32_t width = (uint32_t)(hi - lo);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t k = off + (uint32_t)(64 * (kb >> 1) + 16 * (kb & 1) + r);
                if (!(k < width)) st.s[kb][r] = kNegInf;
            }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (CAP) st.s[kb][r] = cap_score(st.s[kb][r], cap_in2, cap_out);
            mx = fmaxf(mx, st.s[kb][r]);
        }
    if constexpr (CAP) c = 1.f;
    mx = pair_max(mx);
    mx = (mx == kNegInf) ? kNegInf : mx * c;
    // per-row running max, as in the 16-bit kernels: a row's result does not
    // depend on the rows that share its wave
    const bool up = mx > st.m + kRescaleSlack;
    st.need = __any(up);
    const float mnew = up ? mx : st.m;
    st.alpha = (mnew == kNegInf) ? 1.f : fast_exp2(st.m - mnew);
    st.m = mnew;
    const float nm = (mnew == kNegInf) ? 0.f : -mnew;
#pragma unroll
    for (int gp = 0; gp < 2; ++gp)
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) {
            const int kb = 2 * gp + (wd >> 2);
            const int r0 = 4 * (wd & 3);
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sv = st.s[kb][r0 + e];
                pv[e] = fast_exp2(__builtin_fmaf(sv, c, nm));   // c > 0: masked -> 0
            }
            int packed = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
            packed = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], packed, true);
            st.pb[gp][wd] = packed;
            if constexpr (MASKED) {
                // the rounded values back in fp32 (exact), and what they miss
                const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(packed, false);
                const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(packed, true);
                int rest = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0] - h01.x, pv[1] - h01.y, 0, false);
                rest = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2] - h23.x, pv[3] - h23.y, rest, true);
                st.plo[gp][wd] = rest;
            }
        }
    if constexpr (!MASKED) {
        // plo is read only after a masked tile; an empty definition here ends
        // the old remainders' life, so their registers are not held across
        // unmasked tiles (no instruction is emitted)
        asm volatile("" : "=v"(st.plo[0]), "=v"(st.plo[1]));
    }
    st.split = MASKED;
}

__device__ __forceinline__ i32x8_t frag8(const uint8_t* p, uint32_t off) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p + off);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p + (off ^ 16u));
    return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// The 16 bytes at p (any alignment) with bytes nv .. 15 zeroed (nv <= 0: all
// zero), read as the dword-aligned words that hold bytes 0 .. nv-1 only: a
// word holding one of
// them lies inside the tensor (the tensor starts on a 16-byte boundary and
// its size is a multiple of 128 bytes), so nothing past it is touched.
__device__ __forceinline__ u32x4_t load16_any(const uint8_t* p, int nv) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t* wp = reinterpret_cast<const uint32_t*>(a & ~(uintptr_t)3);
    const uint32_t sh = (uint32_t)(a & 3);
    uint32_t wd[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) wd[t] = (nv > 0 && 4 * t < (int)sh + nv) ? wp[t] : 0u;
    u32x4_t r;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // bytes 4t .. 4t+3 of the result: window bytes sh + 4t ..
        uint32_t x = __builtin_amdgcn_alignbyte(wd[t + 1], wd[t], sh);
        const int keep = nv - 4 * t;
        x &= keep >= 4 ? 0xffffffffu : keep <= 0 ? 0u : (0xffffffffu >> (32 - 8 * keep));
        r[t] = x;
    }
    return r;
}

constexpr int kStream8Prefetch = 3;

// The MFMA work of one pipeline phase as a single stream, so the LDS operand
// prefetch runs on across the boundary between the products instead of
// refilling at the start of each:
//   PV: the row sums of P8 (two MFMAs with an all-ones operand, no LDS
//       operand: they cover the first operand reads), then
//       O^T[db] += V^T_tile(db, gp) . P^T(gp), 8 MFMAs (step db*2 + gp,
//       `hook` after each); with LO the remainders plo take two more row-sum
//       MFMAs and one more product per step, on the same V operand;
//   QK: S^T[kb] = K_tile(kb) . Q^T, 8 MFMAs (step t*4 + kb).
// QK runs for every tile, visible keys or not, so the scores are always
// overwritten and the previous tile's are never live across the P.V.
template <bool PV, bool QK, bool LO, class Hook>
__device__ __forceinline__ void mfma_stream8(Fp8Wave& st, const uint8_t* vt, const uint8_t* kt,
                                             const i32x8_t (&q)[2], const Hook& hook) {
    static_assert(PV || QK, "empty stream");
    static_assert(PV || !LO, "remainders belong to a P.V");
    if (PV && st.need) {
#pragma unroll
        for (int db = 0; db < 4; ++db) st.o[db] *= st.alpha;
        st.l *= st.alpha;
        st.need = false;
    }
    const int lane = lane_id();
    const int col = lane & 31, g = lane >> 5;
    // V^T row db*32 + col: its swizzle depends on col only; group gp reads
    // chunks 4gp + 2g and 4gp + 2g + 1 (offset XOR (gp << 6), then XOR 16).
    // K row fp8_krow(kb, col) = kb's block base + rb: its swizzle depends on
    // bits 1, 2, 5 only, which kb does not touch; step t reads chunks
    // 4t + 2g and 4t + 2g + 1.  The empty asm keeps the compiler from
    // hoisting the XORed offsets out of the tile loop.
    const int rb = fp8_krow(0, col);
    uint32_t lov = (uint32_t)(col * D8 + (((2 * g) ^ vswz(col)) << 4));
    uint32_t lok = (uint32_t)(rb * D8 + (((2 * g) ^ kswz(rb)) << 4));
    asm volatile("" : "+v"(lov), "+v"(lok));
    constexpr int NPV = PV ? 8 : 0;
    constexpr int N = NPV + (QK ? 8 : 0);
    auto frag = [&](int i) {
        if (i < NPV) return frag8(vt + (i >> 1) * 32 * D8, lov ^ (uint32_t)((i & 1) << 6));
        const int j = i - NPV, t = j >> 2, kb = j & 3;
        return frag8(kt + (64 * (kb >> 1) + 16 * (kb & 1)) * D8, lok ^ (uint32_t)(t << 6));
    };
    constexpr int PD = kStream8Prefetch;
    i32x8_t a[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) a[i] = frag(i);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PV) {
        const int one4 = 0x38383838;   // four e4m3 1.0
        const i32x8_t ones = {one4, one4, one4, one4, one4, one4, one4, one4};
        st.l = mfma_fp8(ones, st.pb[0], st.l);
        st.l = mfma_fp8(ones, st.pb[1], st.l);
        if constexpr (LO) {
            st.l = mfma_fp8(ones, st.plo[0], st.l);
            st.l = mfma_fp8(ones, st.plo[1], st.l);
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i + PD < N) a[(i + PD) % (PD + 1)] = frag(i + PD);
        __builtin_amdgcn_sched_barrier(0);
        if (i < NPV) {
            st.o[i >> 1] = mfma_fp8(a[i % (PD + 1)], st.pb[i & 1], st.o[i >> 1]);
            if constexpr (LO) st.o[i >> 1] = mfma_fp8(a[i % (PD + 1)], st.plo[i & 1], st.o[i >> 1]);
            hook(i);
        } else {
            const int j = i - NPV;
            st.s[j & 3] = mfma_fp8(a[i % (PD + 1)], q[j >> 2], j < 4 ? f32x16_t{} : st.s[j & 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <class R>
struct Dma8Hook {
    const R& ld;
    typename R::Src sr;
    uint32_t stage;
    int wl;
    bool on;
    __device__ __forceinline__ void operator()(int step) const {
        if (on) ld.dma(step, sr, stage, wl);
    }
};

}  // namespace

template <int NW, bool CAP>
__global__ __launch_bounds__(NW * 64) void k_fp8_prefill(Fp8Params p) {
    static_assert(NW == 8, "two groups of four single-block waves");
    constexpr int BM = NW * 32;
    using R = Ring8;
    static_assert(R::LOADS_PER_TILE == 8, "one load per P.V MFMA");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kStages8 * R::STAGE];
    __shared__ int wave_range[2][NW];

    int b, hg, qt;
    SeqSpan sp;
    if (!map_tile(p.cu_q, p.cu_kv, p.batch, p.n_head_groups, BM >> p.pack_log2, blockIdx.x & 7,
                  blockIdx.x >> 3, b, hg, qt, sp))
        return;
    const int q_start = sp.q_start;
    const int q_len = sp.q_len;
    const int tok0 = qt * (BM >> p.pack_log2);
    const int kv_start = sp.kv_start;
    const int kv_len = sp.kv_len;
    const int h0 = hg << p.pack_log2;
    const int hk = h0 / p.group;
    const float dq = p.descale[0], dk = p.descale[1], dv = p.descale[2];
    const float c_signed = p.scale * dq * dk * kLog2e;
    const bool neg = c_signed < 0.f;
    // at least 1e-30: a masked score (-inf) always gives exp2(-inf) = 0, and
    // a zero scale still weighs every visible key exactly 1
    const float c = fmaxf(fabsf(c_signed), 1e-30f);
    // score cap in log2 units (cap_score), on the descaled score
    const float cap_in2 = CAP ? 2.f * c / p.softcap : 0.f;
    const float cap_out = CAP ? p.softcap * kLog2e : 0.f;

    const int lane = lane_id();
    const int w = wave_id();
    const int col = lane & 31, g = lane >> 5;
    // Waves 0-3 lead, waves 4-7 trail by half a tile; the lead waves alone
    // load the ring, between the MFMAs of their P.V.
    const bool lead = w < NW / 2;
    const int wl = w & (NW / 2 - 1);

    const int r = w * 32 + col;
    const int tok = tok0 + (r >> p.pack_log2);
    const int head = h0 + (r & ((1 << p.pack_log2) - 1));
    const bool valid = tok < q_len;
    i32x8_t q[2];
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
    const int w_lo = wave_min(valid ? lo : 0x7fffffff);
    const int w_hi = wave_max(valid ? hi : -0x7fffffff);
    const int w_lo_max = wave_max(valid ? lo : -0x7fffffff);
    const int w_hi_min = wave_min(valid ? hi : 0x7fffffff);
    const bool w_any = w_hi > w_lo;
    if (lane == 0) {
        wave_range[0][w] = w_any ? w_lo : 0x7fffffff;
        wave_range[1][w] = w_any ? w_hi : -0x7fffffff;
    }
    // The trailing waves' first P.V reads the V^T tile of the last stage
    // before any tile has been loaded there; zeroed, it contributes exactly
    // nothing (uninitialised LDS could hold NaN codes).
    for (int i = threadIdx.x; i < R::TILE / 16; i += NW * 64)
        *reinterpret_cast<u32x4_t*>(ring + (kStages8 - 1) * R::STAGE + R::TILE + 16 * i) =
            u32x4_t{0u, 0u, 0u, 0u};
    __syncthreads();
    int kv_begin = 0x7fffffff, kv_end = -0x7fffffff;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        kv_begin = min(kv_begin, wave_range[0][i]);
        kv_end = max(kv_end, wave_range[1][i]);
    }
    kv_begin = __builtin_amdgcn_readfirstlane(kv_begin & ~15);
    kv_end = __builtin_amdgcn_readfirstlane(kv_end);
    const int n = kv_end > kv_begin ? (kv_end - kv_begin + BN8 - 1) / BN8 : 0;

    const int k_stride = p.num_kv_heads * D8;
    const uint8_t* k_head = p.k + (int64_t)kv_start * k_stride + hk * D8;
    const uint8_t* v_head = p.vt + (int64_t)hk * D8 * p.total_kv + kv_start;
    // Direct loads need 16-byte aligned V^T chunks: every V^T row offset and
    // the sequence start on a 16-key boundary.
    const bool v_aligned = ((p.total_kv & 15) == 0) && ((kv_start & 15) == 0);
    R ld;
    ld.init(lane, wl, k_stride, p.total_kv);
    const uint32_t ring_lds = lds_addr(ring);

    // Loads of the tile at key j0 into the stage at LDS address `stage`:
    // with wave-uniform bases when the tile lies inside the sequence and V^T
    // is aligned (`spread`: the caller issues them one per MFMA), otherwise
    // all at once here with per-lane clamped addresses; rows past kv_len
    // repeat row kv_len - 1 (K) or the last aligned 16-key chunk (V^T), whose
    // probabilities are 0.  An unaligned V^T is gathered from aligned words
    // and written to LDS by the wave (those loads have all returned on exit).
    auto fast = [&](int j0) { return v_aligned && j0 + BN8 <= kv_len; };
    auto src = [&](int j0) {
        return R::Src{k_head + (int64_t)(j0 + 32 * wl) * k_stride,
                      v_head + (int64_t)(32 * wl) * p.total_kv + j0};
    };
    auto issue_all = [&](int j0, uint32_t stage) {
        if (fast(j0)) {
            const R::Src sr = src(j0);
#pragma unroll
            for (int k = 0; k < R::LOADS_PER_TILE; ++k) ld.dma(k, sr, stage, wl);
            return;
        }
        const int last = kv_len - 1;
        // the empty asm keeps the row addresses below from being hoisted out
        // of the tile loop into registers held across it
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (!v_aligned) {
            const uint32_t stage_off = stage - ring_lds;
#pragma unroll
            for (int i = 0; i < R::IPW; ++i) {
                const int d = R::row(ln, wl, i);
                const int key0 = j0 + 16 * R::vchunk(ln, wl, i);
                const int nv = min(max(kv_len - key0, 0), 16);
                const u32x4_t v = load16_any(v_head + (int64_t)d * p.total_kv + key0, nv);
                *reinterpret_cast<u32x4_t*>(ring + stage_off + R::TILE + (wl * R::IPW + i) * 1024 +
                                            16 * ln) = v;
            }
        }
#pragma unroll
        for (int i = 0; i < R::IPW; ++i) {
            const int rr = R::row(ln, wl, i);
            const int key = min(j0 + rr, last);
            dma16(k_head + (int64_t)key * k_stride + R::kchunk(ln, wl, i) * 16,
                  stage + (wl * R::IPW + i) * 1024);
            if (v_aligned) {
                const int key0 = min(j0 + 16 * R::vchunk(ln, wl, i), last & ~15);
                dma16(v_head + (int64_t)rr * p.total_kv + key0,
                      stage + R::TILE + (wl * R::IPW + i) * 1024);
            }
        }
    };
    auto full = [&](int j0) { return j0 >= w_lo_max && j0 + BN8 <= w_hi_min; };

    Fp8Wave st;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db] = f32x16_t{};
    st.l = f32x16_t{};
    st.pb[0] = i32x8_t{};
    st.pb[1] = i32x8_t{};
    st.plo[0] = i32x8_t{};
    st.plo[1] = i32x8_t{};
    st.m = kNegInf;
    st.alpha = 1.f;
    st.need = false;
    st.split = false;

    // Every wave runs every tile: a tile with no visible key for this wave
    // (a causal diagonal) gives P = 0 and leaves m, l and O unchanged.
    auto softmax = [&](int j0) {
        if (full(j0)) softmax8<false, CAP>(st, c, j0, lo, hi, cap_in2, cap_out);
        else softmax8<true, CAP>(st, c, j0, lo, hi, cap_in2, cap_out);
    };

    if (n > 0) {
        // Per tile j: QK(j) -> softmax(j) -> PV(j), the groups offset by half
        // a tile:
        //   phase 1 of tile j: lead softmax(j)               trail PV(j-1), QK(j)
        //   phase 2 of tile j: lead PV(j) + loads, QK(j+1)   trail softmax(j)
        // Tile j+3 goes into the stage of tile j-1, free once phase 1 of
        // tile j is over.
        if (lead) {
#pragma unroll
            for (int k = 0; k < kStages8 - 1; ++k)
                if (k < n) issue_all(kv_begin + k * BN8, ring_lds + k * R::STAGE);
        }
        // Q^T operand (dims 64t + 32g .. +31); a row past the sequence end
        // reads row tok0 (its keys are all masked and it is never stored).
        // Loaded after the ring's first tiles, so the two round trips
        // overlap: the wait for Q below also waits for those tiles, and it
        // leaves no Q load in flight inside the tile loop (where the compiler,
        // which cannot see the ring's direct-to-LDS loads, would wait for it
        // with a count that drains them).
        {
            const uint8_t* qp =
                p.q + ((int64_t)(q_start + (valid ? tok : tok0)) * p.num_heads + head) * D8 + 32 * g;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(qp + 64 * t);
                const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(qp + 64 * t + 16);
                q[t] = i32x8_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                               (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                if (neg) q[t] ^= (int)0x80808080u;   // a negative scale applied to -q
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) asm volatile("" : "+v"(q[t]));
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        block_barrier();
        if (lead) mfma_stream8<false, true, false>(st, ring, ring, q, NoHook{});

        for (int jt = 0; jt < n; ++jt) {
            const int j0 = kv_begin + jt * BN8;
            const uint8_t* st_cur = ring + (jt % kStages8) * R::STAGE;
            const uint8_t* st_prev = ring + ((jt + kStages8 - 1) % kStages8) * R::STAGE;
            const uint8_t* st_next = ring + ((jt + 1) % kStages8) * R::STAGE;
            // phase 1
            if (lead) {
                softmax(j0);
            } else {
                // (at jt == 0 this P.V multiplies P8 = 0 by the zeroed V^T of
                // the last stage: it adds nothing)
                if (st.split)
                    mfma_stream8<true, true, true>(st, st_prev + R::TILE, st_cur, q, NoHook{});
                else
                    mfma_stream8<true, true, false>(st, st_prev + R::TILE, st_cur, q, NoHook{});
            }
            // tile jt+1 must have landed; tile jt+2, issued after it, may stay
            // in flight
            if (lead && jt + 1 < n) {
                if (jt + 2 < n) __builtin_amdgcn_s_waitcnt(vmcnt_imm(R::LOADS_PER_TILE));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            block_barrier();
            // phase 2 (after the last tile the lead's QK reads a stale stage;
            // those scores are never used)
            if (lead) {
                const int j3 = j0 + (kStages8 - 1) * BN8;
                const bool load3 = jt + kStages8 - 1 < n;
                const uint32_t st3 = ring_lds + ((jt + kStages8 - 1) % kStages8) * R::STAGE;
                const bool spread = load3 && fast(j3);
                if (load3 && !spread) issue_all(j3, st3);
                R::Src sr{p.k, p.vt};
                if (spread) sr = src(j3);
                const Dma8Hook<R> hook{ld, sr, st3, wl, spread};
                if (st.split)
                    mfma_stream8<true, true, true>(st, st_cur + R::TILE, st_next, q, hook);
                else
                    mfma_stream8<true, true, false>(st, st_cur + R::TILE, st_next, q, hook);
            } else {
                softmax(j0);
            }
            block_barrier();
        }
        if (!lead) {
            const uint8_t* vt_last = ring + ((n - 1) % kStages8) * R::STAGE + R::TILE;
            if (st.split) mfma_stream8<true, false, true>(st, vt_last, ring, q, NoHook{});
            else mfma_stream8<true, false, false>(st, vt_last, ring, q, NoHook{});
        }
    }

    const float l = st.l[0];
    f32x16_t o_db[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) o_db[db] = st.o[db] * dv;
    // O goes out through this wave's slice of the ring, once the trailing
    // waves' last P.V has read its V^T tile; the slices lie below the last
    // stage's V^T half, which was zeroed before the key loop (with no barrier
    // after it when the loop is empty).
    static_assert(NW * kStoreSliceBytes<D8> <= (kStages8 - 1) * R::STAGE + R::TILE,
                  "output slices clear of the zeroed V^T half");
    block_barrier();
    store_rows_lds<D8, true>(o_db, l, ring + w * kStoreSliceBytes<D8>, [&](int rr) -> uint16_t* {
        const int rw = w * 32 + rr;
        const int tk = tok0 + (rw >> p.pack_log2);
        const int hd = h0 + (rw & ((1 << p.pack_log2) - 1));
        return tk < q_len ? p.out + ((int64_t)(q_start + tk) * p.num_heads + hd) * D8 : nullptr;
    });
    if (valid && p.lse != nullptr && g == 0) {
        const int64_t row = (int64_t)(q_start + tok) * p.num_heads + head;
        p.lse[row] = l > 0.f ? (st.m + __builtin_log2f(l)) * kLn2 : kNegInf;
    }
}

hipError_t launch_fp8_prefill(const Fp8Params& p0, int head_size, int max_seqlen_q,
                              hipStream_t s) {
    if (head_size != D8) return hipErrorInvalidValue;
    // V^T row offsets of one loading wave (32 rows) are 32-bit
    if (p0.total_kv > (1 << 27)) return hipErrorInvalidValue;
    constexpr int NW = 8;
    constexpr int BM = NW * 32;
    Fp8Params p = p0;
    const int tokens_per_tile = BM >> p.pack_log2;
    p.n_qtiles = (max_seqlen_q + tokens_per_tile - 1) / tokens_per_tile;
    const int64_t grid = 8 * tiles_per_xcd(p.batch, p.n_head_groups, p.total_q, max_seqlen_q,
                                           tokens_per_tile);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (p.softcap > 0.f)
        hipLaunchKernelGGL((k_fp8_prefill<NW, true>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
    else
        hipLaunchKernelGGL((k_fp8_prefill<NW, false>), dim3((unsigned)grid), dim3(NW * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace attn
