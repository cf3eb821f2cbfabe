// Varlen attention backward on gfx950: dQ, dK, dV from Q, K, V, the forward
// output O, the upstream gradient dO and the forward's saved logsumexp (the
// LSE output the blt issue's FlexAttention kernel options turn on; the
// vllm-project/flash-attention "Rope dim" review shows the varlen function's
// backward returning dq, dk, dv).
//
// With P = exp(scale * Q K^T - LSE) (masked entries 0) and
// delta = rowsum(dO * O) = rowsum(dP * P):
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),
//     dQ = scale dS K,  dK = scale dS^T Q.
// Two kernels, no atomics:
//   k_bwd_dq     a workgroup owns 128 query rows of one head (32 per wave,
//                one per lane column, Q and dO in registers as the B
//                operands); it computes each row's delta from its dO and O
//                (stored for the second kernel) and streams 64-key K / V
//                tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T;
//   k_bwd_dkdv16 a workgroup owns 128 keys of one kv head, 16 per wave (K
//                and V rows in registers), and streams 64-row Q / dO tiles of
//                every query head of the group: S = Q K^T, dP = dO V^T, then
//                dV^T += dO^T P and dK^T += Q^T dS on 16x16x32 MFMA tiles --
//                the group's heads sum in registers.
// Both stream kernels use the two MFMA patterns of the forward: rows of an
// LDS tile against a register operand (the S^T = K Q^T product), and the
// transposed LDS read against packed 16-bit accumulators (the P.V product),
// on tiles in the same swizzled row-major LDS layout.  Tiles arrive by direct
// global->LDS loads and are double-buffered: the next tile's loads are in
// flight while the current one is used.

#include "device_common.h"
#include "kernels.h"
#include "ring.h"

namespace attn {

namespace {

constexpr int kBwdTile = 64;    // rows of a streamed tile
constexpr int kBwdRows = 128;   // rows a workgroup owns (4 waves x 32)

// MFMA steps 0 .. N-1 with their A operands read PD steps ahead through a
// small register ring (the forward's prefetch queue): without it the
// compiler reuses one operand register and every MFMA waits out a full LDS
// read.  sched_barrier pins the order.
template <int N, int PD, class Frag, class Op>
__device__ __forceinline__ void mfma_queue(const Frag& frag, const Op& op) {
    constexpr int P = PD < N ? PD : N;
    u32x4_t a[P + 1];
#pragma unroll
    for (int i = 0; i < P; ++i) a[i] = frag(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i + P < N) a[(i + P) % (P + 1)] = frag(i + P);
        __builtin_amdgcn_sched_barrier(0);
        op(i, a[i % (P + 1)]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

constexpr int kBwdPrefetch = 4;

// Chunk swizzle of the dK/dV kernel's Q and dO tiles.  Its two reads:
//   * 16-byte operand reads (16 lanes per LDS cycle): 16 aligned rows, one
//     logical chunk -> the swizzle must be a bijection on each aligned
//     16 rows (per row parity at D = 64, where a row spans half the banks);
//   * transposed 8-byte reads: lane quarter q reads rows 4q .. 4q+3 of an
//     aligned 16, two neighbouring chunks {2m, 2m+1} per row, and the chunk
//     pair m ^ (s >> 1) must differ between the rows served in one cycle --
//     whether a cycle pairs quarters {0, 1} or {0, 2}, i.e. s >> 1 distinct
//     on rows {0..7} and on rows {0..3, 8..11} (and their complements; per
//     parity at D = 64).
// With r = b3 b2 b1 b0, s >> 1 takes the low row bits (b1 b0; b1 at D = 64)
// and b2 ^ b3, and b3 fills the last bit.  swz<D> meets the first condition
// only (rows r and r + 4 share a pair).
template <int D>
__device__ __forceinline__ int swz_dkdv(int r) {
    const int x23 = ((r >> 2) ^ (r >> 3)) & 1, b3 = (r >> 3) & 1;
    if constexpr (D == 128) return (((r & 3) | (x23 << 2)) << 1) | b3;
    else return ((((r >> 1) & 1) | (x23 << 1)) << 1) | b3;
}

// 64 rows x D of a [tokens, heads, D] tensor straight into the swizzled LDS
// tile layout with direct global->LDS loads, shared by the NW waves (wave w
// issues its share).  Lane l of a 1 KB load lands at byte 16 l of it:
// row i*RPI + l/CPR, physical chunk l % CPR, which holds the logical chunk
// (l % CPR) ^ sw(row), sw = swz_dkdv<D> when DKDV, else swz<D>.  Rows at or
// past n read row n - 1 (n >= 1).  The caller waits for the loads (vmcnt)
// before the barrier that publishes them.
template <int D, int NW = 4, bool DKDV = false>
__device__ __forceinline__ void dma_rows(const uint16_t* base, int64_t stride, int r0, int n,
                                         uint32_t tile, int w, int lane) {
    constexpr int CPR = D / 8, RPI = 64 / CPR, NI = kBwdTile / RPI;
    static_assert(NI % NW == 0, "a tile's loads split evenly over the waves");
#pragma unroll
    for (int k = 0; k < NI / NW; ++k) {
        const int i = w * (NI / NW) + k;
        const int row = i * RPI + lane / CPR;
        const int c = (lane % CPR) ^ (DKDV ? swz_dkdv<D>(row) : swz<D>(row));
        const int rr = min(max(r0 + row, 0), n - 1);
        dma16(base + rr * stride + c * 8, tile + i * 1024);
    }
}

// Two row products of one 32-row block kb in one queue:
//   x = tile_x rows kb*32.. . bx,  y = tile_y rows kb*32.. . by
// -- the S^T = K Q^T pattern: rows of the LDS tile against this lane
// column's register row (dims 16t + 8g .. +7 in b[t]).
template <int D, bool BF16>
__device__ __forceinline__ void rows_dot2_block(f32x16_t& x, f32x16_t& y, const uint8_t* tx,
                                                const uint8_t* ty, const u32x4_t (&bx)[D / 16],
                                                const u32x4_t (&by)[D / 16], int kb) {
    constexpr int ROWB = 2 * D;
    constexpr int H = D / 16;
    const int lane = lane_id(), col = lane & 31, g = lane >> 5;
    uint32_t lok = (uint32_t)(kb * 32 * ROWB + col * ROWB + ((g ^ swz<D>(col)) << 4));
    asm volatile("" : "+v"(lok));
    auto frag = [&](int i) {
        const int t = i % H;
        return *reinterpret_cast<const u32x4_t*>((i < H ? tx : ty) + (lok ^ (uint32_t)(t << 5)));
    };
    auto op = [&](int i, const u32x4_t& a) {
        const int t = i % H;
        if (i < H) x = mfma32<BF16>(a, bx[t], t == 0 ? f32x16_t{} : x);
        else y = mfma32<BF16>(a, by[t], t == 0 ? f32x16_t{} : y);
    };
    mfma_queue<2 * H, kBwdPrefetch>(frag, op);
}

// The block-kb part of a column accumulation: y[db] += tile^T (rows
// kb*32..) . X, with X the packed 16-bit accumulators of a row product
// (rows = tile rows) -- the P.V pattern with the transposed LDS read.
template <int D, bool BF16>
__device__ __forceinline__ void cols_acc_block(f32x16_t (&y)[D / 32], const uint8_t* tile,
                                               const u32x4_t (&xb)[2], int kb) {
    constexpr int H = (D / 32) * 2;
    uint32_t lo0, hi0;
    pv_offsets<D>(lo0, hi0);
    asm volatile("" : "+v"(lo0), "+v"(hi0));
    auto frag = [&](int i) {
        return pv_frag<D, kBwdTile>(tile, lo0, hi0, (i / 2) * 4 + kb * 2 + i % 2);
    };
    auto op = [&](int i, const u32x4_t& a) { y[i / 2] = mfma32<BF16>(a, xb[i % 2], y[i / 2]); };
    mfma_queue<H, kBwdPrefetch>(frag, op);
}

// Accumulator values 8tp .. 8tp+7 of block kb packed as the B operand.
template <bool BF16>
__device__ __forceinline__ void pack_block(const float (&v)[16], u32x4_t (&xb)[2]) {
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
        u32x4_t w;
        w.x = pack2<BF16>(v[8 * tp + 0], v[8 * tp + 1]);
        w.y = pack2<BF16>(v[8 * tp + 2], v[8 * tp + 3]);
        w.z = pack2<BF16>(v[8 * tp + 4], v[8 * tp + 5]);
        w.w = pack2<BF16>(v[8 * tp + 6], v[8 * tp + 7]);
        xb[tp] = w;
    }
}

// Write acc^T (rows = dims, column = lane's column) times f to one D-long row.
template <int D, bool BF16>
__device__ __forceinline__ void store_cols(const f32x16_t (&acc)[D / 32], float f, uint16_t* row) {
    const int g = lane_id() >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            u32x2_t w;
            w.x = pack2<BF16>(acc[db][4 * rq + 0] * f, acc[db][4 * rq + 1] * f);
            w.y = pack2<BF16>(acc[db][4 * rq + 2] * f, acc[db][4 * rq + 3] * f);
            *reinterpret_cast<u32x2_t*>(row + db * 32 + 8 * rq + 4 * g) = w;
        }
}

template <bool BF16>
__device__ __forceinline__ f32x2_t unpack16(uint32_t w) {
    if constexpr (BF16) {
        return f32x2_t{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
    } else {
        return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
    }
}

// P and dS of one score.  s: raw q.k; lse2: the row's LSE in log2 units.
// Without a cap the log2 score is s * c.  With a cap (CAP) the score is
// cap tanh(scale s / cap): t = 1 - 2 / (1 + 2^(s * in2)) with the signed
// in2 = 2 log2(e) scale / cap (2^(.) overflowing to +inf gives t = 1, to 0
// gives t = -1), the log2 score is out * t with out = cap log2(e), and dS
// takes the derivative 1 - t^2.
template <bool CAP>
__device__ __forceinline__ float prob_ds(float s, float dp, float lse2, float delta,
                                         const BwdParams& p, float& pr) {
    if constexpr (CAP) {
        const float e = fast_exp2(s * p.cap_in2);
        const float t = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + e), 1.f);
        pr = fast_exp2(__builtin_fmaf(t, p.cap_out, -lse2));
        return pr * (dp - delta) * __builtin_fmaf(-t, t, 1.f);
    } else {
        pr = fast_exp2(__builtin_fmaf(s, p.c, -lse2));
        return pr * (dp - delta);
    }
}

template <int D, bool BF16, bool CAP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_bwd_dq(BwdParams p) {
    constexpr int TILE = kBwdTile * 2 * D;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2 * TILE];   // [buffer][K, V]
    __shared__ int wave_range[2][4];
    // XCD-aware order: workgroup i runs on XCD i % 8; every workgroup of a
    // (sequence, kv head) unit -- its query heads' row tiles, which stream
    // the same K / V tiles -- lands on one XCD and shares its L2
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int per = p.group * p.n_qt;
    const int u = xcd + 8 * (j / per), rj = j % per;
    if (u >= p.batch * p.num_kv_heads) return;
    const int b = u / p.num_kv_heads;
    const int h = (u % p.num_kv_heads) * p.group + rj / p.n_qt;
    const int q_start = p.cu_q[b], q_len = p.cu_q[b + 1] - q_start;
    const int row0 = (rj % p.n_qt) * kBwdRows;
    if (row0 >= q_len) return;
    const int kv_start = p.cu_kv[b], kv_len = p.cu_kv[b + 1] - kv_start;
    const int hk = h / p.group;
    const int lane = lane_id(), w = wave_id();
    const int col = lane & 31, g = lane >> 5;
    const int r = row0 + w * 32 + col;
    const bool valid = r < q_len;
    const int rr = valid ? r : q_len - 1;
    const int64_t qrow = (int64_t)(q_start + rr) * p.num_heads + h;

    u32x4_t qv[D / 16], dov[D / 16], ov[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
        qv[t] = *reinterpret_cast<const u32x4_t*>(p.q + qrow * D + 16 * t + 8 * g);
        dov[t] = *reinterpret_cast<const u32x4_t*>(p.dout + qrow * D + 16 * t + 8 * g);
        ov[t] = *reinterpret_cast<const u32x4_t*>(p.out + qrow * D + 16 * t + 8 * g);
    }
    const float lse2 = p.lse[qrow] * kLog2e;
    // delta = sum_d dO * O in fp32: this lane's half row (dims 16t + 8g ..
    // + 7), then the other half from lane l ^ 32; stored for the dK/dV kernel
    float dpart = 0.f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x2_t fo = unpack16<BF16>(ov[t][e]), fd = unpack16<BF16>(dov[t][e]);
            dpart = __builtin_fmaf(fo.x, fd.x, dpart);
            dpart = __builtin_fmaf(fo.y, fd.y, dpart);
        }
    const float dlt = pair_sum(dpart);
    if (valid && g == 0) p.delta[qrow] = dlt;
    // this row's visible keys [lo, hi), as in the forward
    int lo = 0, hi = 0;
    if (valid) {
        hi = kv_len;
        if (p.mask & kMaskCausal) hi = min(hi, r + (kv_len - q_len) + 1);
        if (p.mask & kMaskPatch) hi = min(hi, p.q_ids[q_start + r] + 1);
        if (p.mask & kMaskDocument) {
            const int doc = p.q_ids[q_start + r];
            lo = lower_bound_i32(p.kv_ids + kv_start, kv_len, doc);
            hi = min(hi, upper_bound_i32(p.kv_ids + kv_start, kv_len, doc));
        }
        if (p.window > 0) lo = max(lo, r + (kv_len - q_len) - p.window + 1);
        if (hi < lo) hi = lo;
    }
    const bool any = valid && hi > lo;
    const int w_lo = wave_min(any ? lo : 0x7fffffff);
    const int w_hi = wave_max(any ? hi : -1);
    // a tile inside every row's interval needs no mask (rows past the
    // sequence count as empty, so a wave holding any is never "full")
    const int w_lo_max = wave_max(valid ? lo : 0x7fffffff);
    const int w_hi_min = wave_min(valid ? hi : -1);
    if (lane == 0) {
        wave_range[0][w] = w_lo;
        wave_range[1][w] = w_hi;
    }
    __syncthreads();
    int kv_begin = 0x7fffffff, kv_end = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kv_begin = min(kv_begin, wave_range[0][i]);
        kv_end = max(kv_end, wave_range[1][i]);
    }
    kv_begin = __builtin_amdgcn_readfirstlane(kv_begin);
    kv_end = __builtin_amdgcn_readfirstlane(kv_end);
    const int n_t = kv_end > kv_begin ? (kv_end - kv_begin + kBwdTile - 1) / kBwdTile : 0;

    f32x16_t acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16_t{};
    if (n_t > 0) {
        const int64_t stride = (int64_t)p.num_kv_heads * D;
        const uint16_t* kbase = p.k + ((int64_t)kv_start * p.num_kv_heads + hk) * D;
        const uint16_t* vbase = p.v + ((int64_t)kv_start * p.num_kv_heads + hk) * D;
        const uint32_t lds0 = lds_addr(lds);
        auto fetch = [&](int j0, int bf) {
            const uint32_t t = lds0 + bf * 2 * TILE;
            dma_rows<D>(kbase, stride, j0, kv_len, t, w, lane);
            dma_rows<D>(vbase, stride, j0, kv_len, t + TILE, w, lane);
        };
        fetch(kv_begin, 0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        for (int it = 0; it < n_t; ++it) {
            const int j0 = kv_begin + it * kBwdTile;
            const uint8_t* kt = lds[it & 1];
            const uint8_t* vt = kt + TILE;
            if (it + 1 < n_t) fetch(j0 + kBwdTile, (it + 1) & 1);
            // this wave's rows against keys j0 .. j0 + 63: none visible (skip),
            // all visible (no mask), or some
            const bool skip = j0 >= w_hi || j0 + kBwdTile <= w_lo;
            if (!skip) {
                const bool full = j0 >= w_lo_max && j0 + kBwdTile <= w_hi_min;
                // the tile's two 32-key blocks one after the other, so only one
                // block's S, dP and dS are live at a time
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    f32x16_t s1, dp1;
                    rows_dot2_block<D, BF16>(s1, dp1, kt, vt, qv, dov, kb);
                    float ds[16];
                    float pr;
                    if (full) {
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            ds[e] = prob_ds<CAP>(s1[e], dp1[e], lse2, dlt, p, pr);
                    } else {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = j0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                            const float d = prob_ds<CAP>(s1[e], dp1[e], lse2, dlt, p, pr);
                            ds[e] = (key >= lo && key < hi) ? d : 0.f;
                        }
                    }
                    u32x4_t xb[2];
                    pack_block<BF16>(ds, xb);
                    cols_acc_block<D, BF16>(acc, kt, xb, kb);
                }
            }
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
        }
    }
    if (valid) store_cols<D, BF16>(acc, p.scale, p.dq + qrow * D);
}

// 16x16x32 MFMA on 8 packed 16-bit values per lane: lane l holds row (A) or
// column (B) l % 16 and k-slots 8 (l / 16) .. +7; the 16x16 accumulator
// gives lane l column l % 16, rows 4 (l / 16) + r in register r.
template <bool BF16>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
}

// The dK/dV kernel with 16 keys per wave on 16x16x32 MFMA tiles: eight waves
// own the workgroup's 128 keys, two per SIMD (the accumulators of a 16-key
// slice, 2 x D/16 x 4 registers, leave room for a second wave).  Per 64-row
// Q / dO tile, for each of the four 16-row blocks: S = Q K^T and dP = dO V^T
// (Q / dO rows from LDS as A, this lane column's K / V row in registers as
// B); then dV^T += dO^T P and dK^T += Q^T dS over the 64 rows in two 32-row
// steps, with P and dS packed from the accumulators of blocks 2st, 2st + 1
// as the B operand (k-slots 0..3: rows 32st + 4g + r, 4..7: rows
// 32st + 16 + 4g + r for lane group g) and dO^T / Q^T read transposed from
// LDS in the same row order.
template <int D, bool BF16, bool CAP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_bwd_dkdv16(
    BwdParams p) {
    constexpr int NW = 8;
    constexpr int ROWB = 2 * D;
    constexpr int TILE = kBwdTile * ROWB;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2 * TILE];   // [buffer][Q, dO]
    __shared__ __attribute__((aligned(16))) float rows_lse2[2][kBwdTile];
    __shared__ __attribute__((aligned(16))) float rows_delta[2][kBwdTile];
    __shared__ __attribute__((aligned(16))) int rows_lo[2][kBwdTile];
    __shared__ __attribute__((aligned(16))) int rows_hi[2][kBwdTile];
    __shared__ int tile_ext[2][4];   // per tile: max lo, min hi, min lo, max hi
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int u = xcd + 8 * (j / p.n_kt);
    if (u >= p.batch * p.num_kv_heads) return;
    const int b = u / p.num_kv_heads, hk = u % p.num_kv_heads;
    const int kv_start = p.cu_kv[b], kv_len = p.cu_kv[b + 1] - kv_start;
    const int k0 = (j % p.n_kt) * kBwdRows;
    if (k0 >= kv_len) return;
    const int q_start = p.cu_q[b], q_len = p.cu_q[b + 1] - q_start;
    const int off = kv_len - q_len;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int c16 = lane & 15, g = lane >> 4;
    const int key = k0 + w * 16 + c16;
    const bool kvalid = key < kv_len;
    const int kk = kvalid ? key : kv_len - 1;
    const int64_t krow = (int64_t)(kv_start + kk) * p.num_kv_heads + hk;

    u32x4_t kr[D / 32], vr[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
        kr[t] = *reinterpret_cast<const u32x4_t*>(p.k + krow * D + 32 * t + 8 * g);
        vr[t] = *reinterpret_cast<const u32x4_t*>(p.v + krow * D + 32 * t + 8 * g);
    }
    const bool causal = p.mask & kMaskCausal;
    const int wk_lo = k0 + w * 16;
    const int wk_hi = min(wk_lo + 16, kv_len);   // exclusive

    int qlo = 0, qhi = q_len;
    if (causal) qlo = max(qlo, k0 - off);
    if (p.window > 0) qhi = min(qhi, k0 + kBwdRows - 1 - off + p.window);
    const int n_qt = qhi > qlo ? (qhi - qlo + kBwdTile - 1) / kBwdTile : 0;
    const int n_t = n_qt * p.group;

    f32x4_t dk[D / 16], dv[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) dk[db] = dv[db] = f32x4_t{};
    if (n_t > 0 && q_len > 0) {
        const int64_t stride = (int64_t)p.num_heads * D;
        // Query tiles are aligned to qhi and taken from the top down, with
        // the group's heads innermost: the workgroups of one kv head, which
        // run together on one XCD, then read the same Q / dO tiles at about
        // the same time, and all but the first find them in the L2.  The
        // bottom tile may reach below qlo (rows that see none of these keys)
        // or below row 0 (rows that do not exist: loads clamped, masked).
        auto head_of = [&](int it) { return hk * p.group + it % p.group; };
        auto row0_of = [&](int it) { return qhi - kBwdTile * (it / p.group + 1); };
        const uint32_t lds0 = lds_addr(lds);
        auto load = [&](int it, int bf) {
            const int h = head_of(it), j0 = row0_of(it);
            const int64_t base = (int64_t)q_start * p.num_heads + h;
            const uint32_t t = lds0 + bf * 2 * TILE;
            dma_rows<D, NW, true>(p.q + base * D, stride, j0, q_len, t, w, lane);
            dma_rows<D, NW, true>(p.dout + base * D, stride, j0, q_len, t + TILE, w, lane);
        };
        // per-row values of tile it into buffer bf (wave 0), in two parts:
        // rows_dma issues the row's LSE and delta as direct global->LDS loads
        // (one 4-byte load per row; rows past the sequence read its last
        // row), together with the tile's Q / dO loads, so their latency is
        // spent under a tile of MFMAs; rows_fin, a tile later, waits for
        // them, scales the LSE to log2 units, zeroes rows past the sequence
        // and computes the row's visible keys [lo, hi) as in the forward
        // (empty past the sequence) and the tile's extreme bounds
        auto rows_dma = [&](int it, int bf) {
            if (tid < kBwdTile) {
                const int h = head_of(it), q = row0_of(it) + tid;
                const int64_t i = (int64_t)(q_start + min(max(q, 0), q_len - 1)) * p.num_heads + h;
                dma4(p.lse + i, lds_addr(&rows_lse2[bf][0]));
                dma4(p.delta + i, lds_addr(&rows_delta[bf][0]));
            }
        };
        auto rows_fin = [&](int it, int bf) {
            if (tid < kBwdTile) {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                asm volatile("" ::: "memory");   // LDS reads below stay after the wait
                const int q = row0_of(it) + tid;
                const bool in = q >= 0 && q < q_len;
                rows_lse2[bf][tid] = in ? rows_lse2[bf][tid] * kLog2e : 0.f;
                rows_delta[bf][tid] = in ? rows_delta[bf][tid] : 0.f;
                int lo = 0, hi = 0;
                if (in) {
                    hi = kv_len;
                    if (causal) hi = min(hi, q + off + 1);
                    if (p.mask & kMaskPatch) hi = min(hi, p.q_ids[q_start + q] + 1);
                    if (p.mask & kMaskDocument) {
                        const int d = p.q_ids[q_start + q];
                        lo = lower_bound_i32(p.kv_ids + kv_start, kv_len, d);
                        hi = min(hi, upper_bound_i32(p.kv_ids + kv_start, kv_len, d));
                    }
                    if (p.window > 0) lo = max(lo, q + off - p.window + 1);
                    if (hi < lo) hi = lo;
                }
                rows_lo[bf][tid] = lo;
                rows_hi[bf][tid] = hi;
                const int lo_max = wave_max(lo), hi_min = wave_min(hi);
                const bool ne = hi > lo;
                const int lo_min = wave_min(ne ? lo : 0x7fffffff);
                const int hi_max = wave_max(ne ? hi : -1);
                if (tid == 0) {
                    tile_ext[bf][0] = lo_max;
                    tile_ext[bf][1] = hi_min;
                    tile_ext[bf][2] = lo_min;
                    tile_ext[bf][3] = hi_max;
                }
            }
        };
        // A-operand lane offsets.  Rows of an S / dP block: row 16 qb + c16,
        // logical chunk 4t + g (its swizzle depends on the row mod 16 only).
        uint32_t arow = (uint32_t)(c16 * ROWB);
        const int asw = swz_dkdv<D>(c16);
        asm volatile("" : "+v"(arow));
        load(0, 0);
        rows_dma(0, 0);
        rows_fin(0, 0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        for (int it = 0; it < n_t; ++it) {
            const int bf = it & 1;
            const uint8_t* qt = lds[bf];
            const uint8_t* dt = qt + TILE;
            const bool more = it + 1 < n_t;
            if (more) {
                load(it + 1, bf ^ 1);
                rows_dma(it + 1, bf ^ 1);
            }
            const int lo_max = tile_ext[bf][0], hi_min = tile_ext[bf][1];
            const int lo_min = tile_ext[bf][2], hi_max = tile_ext[bf][3];
            const bool skip = wk_hi <= wk_lo || wk_hi <= lo_min || wk_lo >= hi_max;
            if (!skip) {
                const bool full = lo_max <= wk_lo && hi_min >= wk_hi && wk_hi - wk_lo == 16;
                f32x4_t s4[4], dp4[4];
                {
                    constexpr int H = 4 * (D / 32);   // steps per product (qb, t)
                    auto frag = [&](int i) {
                        const int jj = i % H, qb = jj / (D / 32), t = jj % (D / 32);
                        const uint8_t* tile = i < H ? qt : dt;
                        return *reinterpret_cast<const u32x4_t*>(
                            tile + qb * 16 * ROWB + arow + (((4 * t + g) ^ asw) << 4));
                    };
                    auto op = [&](int i, const u32x4_t& a) {
                        const int jj = i % H, qb = jj / (D / 32), t = jj % (D / 32);
                        if (i < H) s4[qb] = mfma16<BF16>(a, kr[t], t == 0 ? f32x4_t{} : s4[qb]);
                        else dp4[qb] = mfma16<BF16>(a, vr[t], t == 0 ? f32x4_t{} : dp4[qb]);
                    };
                    mfma_queue<2 * H, kBwdPrefetch>(frag, op);
                }
                float pv[4][4], dsv[4][4];
#pragma unroll
                for (int qb = 0; qb < 4; ++qb) {
                    const int tr = qb * 16 + 4 * g;   // tile rows tr .. tr+3
                    const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(&rows_lse2[bf][tr]);
                    const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&rows_delta[bf][tr]);
                    if (full) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            dsv[qb][r] = prob_ds<CAP>(s4[qb][r], dp4[qb][r], l4[r], d4[r], p, pv[qb][r]);
                    } else {
                        const i32x4_t lo4 = *reinterpret_cast<const i32x4_t*>(&rows_lo[bf][tr]);
                        const i32x4_t hi4 = *reinterpret_cast<const i32x4_t*>(&rows_hi[bf][tr]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool vis = kvalid && key >= lo4[r] && key < hi4[r];
                            float pr;
                            const float d = prob_ds<CAP>(s4[qb][r], dp4[qb][r], l4[r], d4[r], p, pr);
                            pv[qb][r] = vis ? pr : 0.f;
                            dsv[qb][r] = vis ? d : 0.f;
                        }
                    }
                }
                u32x4_t pbp[2], pbs[2];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    pbp[st] = u32x4_t{pack2<BF16>(pv[2 * st][0], pv[2 * st][1]),
                                      pack2<BF16>(pv[2 * st][2], pv[2 * st][3]),
                                      pack2<BF16>(pv[2 * st + 1][0], pv[2 * st + 1][1]),
                                      pack2<BF16>(pv[2 * st + 1][2], pv[2 * st + 1][3])};
                    pbs[st] = u32x4_t{pack2<BF16>(dsv[2 * st][0], dsv[2 * st][1]),
                                      pack2<BF16>(dsv[2 * st][2], dsv[2 * st][3]),
                                      pack2<BF16>(dsv[2 * st + 1][0], dsv[2 * st + 1][1]),
                                      pack2<BF16>(dsv[2 * st + 1][2], dsv[2 * st + 1][3])};
                }
                {
                    // transposed reads: lane 4e + qq of group g points at row
                    // 32st + 16rd + 4g + e, columns 16db + 4qq .. +3; output
                    // lane c16 receives that row quad of column 16db + c16
                    const int e = c16 >> 2, qq = c16 & 3;
                    constexpr int H = (D / 16) * 2;   // steps per product (db, st)
                    auto tr8 = [&](const uint8_t* tile, int row, int col) {
                        return ds_read_tr16(tile + row * ROWB + ((((col >> 3) ^ swz_dkdv<D>(row))) << 4) +
                                            (col & 7) * 2);
                    };
                    auto frag = [&](int i) {
                        const int jj = i % H, db = jj / 2, st = jj % 2;
                        const uint8_t* tile = i < H ? dt : qt;
                        const int r0 = 32 * st + 4 * g + e, col = 16 * db + 4 * qq;
                        const u32x2_t x0 = tr8(tile, r0, col);
                        const u32x2_t x1 = tr8(tile, r0 + 16, col);
                        return u32x4_t{x0.x, x0.y, x1.x, x1.y};
                    };
                    auto op = [&](int i, const u32x4_t& a) {
                        const int jj = i % H, db = jj / 2, st = jj % 2;
                        if (i < H) dv[db] = mfma16<BF16>(a, pbp[st], dv[db]);
                        else dk[db] = mfma16<BF16>(a, pbs[st], dk[db]);
                    };
                    mfma_queue<2 * H, kBwdPrefetch>(frag, op);
                }
            }
            if (more) rows_fin(it + 1, bf ^ 1);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
        }
    }
    if (kvalid) {
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            u32x2_t a, c;
            a.x = pack2<BF16>(dk[db][0] * p.scale, dk[db][1] * p.scale);
            a.y = pack2<BF16>(dk[db][2] * p.scale, dk[db][3] * p.scale);
            c.x = pack2<BF16>(dv[db][0], dv[db][1]);
            c.y = pack2<BF16>(dv[db][2], dv[db][3]);
            *reinterpret_cast<u32x2_t*>(p.dk + krow * D + 16 * db + 4 * g) = a;
            *reinterpret_cast<u32x2_t*>(p.dv + krow * D + 16 * db + 4 * g) = c;
        }
    }
}

template <int D, bool BF16, bool CAP>
hipError_t launch_bwd_cfg(const BwdParams& p, int max_seqlen_q, int max_seqlen_kv, hipStream_t s) {
    hipError_t e = hipSuccess;
    BwdParams q = p;
    q.n_qt = (max_seqlen_q + kBwdRows - 1) / kBwdRows;
    q.n_kt = (max_seqlen_kv + kBwdRows - 1) / kBwdRows;
    const int64_t slots = 8 * (((int64_t)p.batch * p.num_kv_heads + 7) / 8);   // units, padded
    const int64_t gq = slots * p.group * q.n_qt, gk = slots * q.n_kt;
    if (gq > 0x7fffffff || gk > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (gq > 0) {
        hipLaunchKernelGGL((k_bwd_dq<D, BF16, CAP>), dim3((unsigned)gq), dim3(256), 0, s, q);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (gk > 0) {
        hipLaunchKernelGGL((k_bwd_dkdv16<D, BF16, CAP>), dim3((unsigned)gk), dim3(512), 0, s, q);
        e = hipGetLastError();
    }
    return e;
}

template <int D, bool BF16>
hipError_t launch_bwd_cap(const BwdParams& p, int max_seqlen_q, int max_seqlen_kv, hipStream_t s) {
    return p.cap_out > 0.f ? launch_bwd_cfg<D, BF16, true>(p, max_seqlen_q, max_seqlen_kv, s)
                           : launch_bwd_cfg<D, BF16, false>(p, max_seqlen_q, max_seqlen_kv, s);
}

}  // namespace

hipError_t launch_varlen_bwd(const BwdParams& p, int head_size, bool bf16, int max_seqlen_q,
                             int max_seqlen_kv, hipStream_t s) {
    if (head_size == 128)
        return bf16 ? launch_bwd_cap<128, true>(p, max_seqlen_q, max_seqlen_kv, s)
                    : launch_bwd_cap<128, false>(p, max_seqlen_q, max_seqlen_kv, s);
    if (head_size == 64)
        return bf16 ? launch_bwd_cap<64, true>(p, max_seqlen_q, max_seqlen_kv, s)
                    : launch_bwd_cap<64, false>(p, max_seqlen_q, max_seqlen_kv, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
