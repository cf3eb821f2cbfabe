// cu_seqlens (exclusive scan) and reshape_and_cache (paged scatter) on gfx950.
//
// Both are the preprocessing steps of the onnxruntime PR "[CUDA]
// PagedAttention: add SM<80 fp16 fallback via memory-efficient attention"
// (section Implementation, step 1: LaunchGetCumulativeSeqlensKV and
// ReshapeAndCache).

#include "device_common.h"
#include "kernels.h"

namespace attn {

// One workgroup scans the whole array in 1024-element chunks, carrying the
// running total between chunks.
__global__ __launch_bounds__(1024) void k_cu_seqlens(const int32_t* __restrict__ lens,
                                                      int32_t* __restrict__ cu, int n) {
    __shared__ int wsum[16];
    const int lane = lane_id(), w = wave_id();
    int carry = 0;
    if (threadIdx.x == 0) cu[0] = 0;
    for (int base = 0; base < n; base += 1024) {
        const int i = base + threadIdx.x;
        int x = i < n ? lens[i] : 0;
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
            const int y = __shfl_up(x, s, 64);
            if (lane >= s) x += y;
        }
        if (lane == 63) wsum[w] = x;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int v = wsum[k];
            before += (k < w) ? v : 0;
            total += v;
        }
        if (i < n) cu[i + 1] = carry + before + x;
        carry += total;
        __syncthreads();
    }
}

hipError_t launch_cu_seqlens(const int32_t* seqlens, int32_t* cu, int batch, hipStream_t s) {
    hipLaunchKernelGGL(k_cu_seqlens, dim3(1), dim3(1024), 0, s, seqlens, cu, batch);
    return hipGetLastError();
}

// One wave copies one new token's K and V rows (num_kv_heads * head_size
// elements each, `chunks` 16-byte pieces) into the cache slot of its
// position; waves stride over the tokens.
__global__ __launch_bounds__(256) void k_reshape_and_cache(
    const uint8_t* __restrict__ k, const uint8_t* __restrict__ v, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int32_t* __restrict__ block_table, int mbps,
    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ cu_kv, int batch,
    int total_new, int chunks, int bs_log2) {
    const int lane = lane_id();
    const int waves = gridDim.x * 4;
    for (int t = blockIdx.x * 4 + wave_id(); t < total_new; t += waves) {
        // sequence of token t: last b with cu_new[b] <= t
        int lo = 0, hi = batch;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu_new[mid] <= t) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int n_new = cu_new[b + 1] - cu_new[b];
        const int kv_len = cu_kv[b + 1] - cu_kv[b];
        const int pos = kv_len - n_new + (t - cu_new[b]);
        const int64_t page = block_table[(int64_t)b * mbps + (pos >> bs_log2)];
        const int64_t dst = ((page << bs_log2) + (pos & ((1 << bs_log2) - 1))) * chunks;
        const int64_t src = (int64_t)t * chunks;
        for (int c = lane; c < chunks; c += 64) {
            const u32x4_t kv = reinterpret_cast<const u32x4_t*>(k)[src + c];
            const u32x4_t vv = reinterpret_cast<const u32x4_t*>(v)[src + c];
            reinterpret_cast<u32x4_t*>(k_cache)[dst + c] = kv;
            reinterpret_cast<u32x4_t*>(v_cache)[dst + c] = vv;
        }
    }
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* block_table, int mbps, const int32_t* cu_new,
                                    const int32_t* cu_kv, int batch, int total_new,
                                    int row_bytes, int bs_log2, hipStream_t s) {
    const int chunks = row_bytes / 16;
    int blocks = (total_new + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_reshape_and_cache, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v),
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       block_table, mbps, cu_new, cu_kv, batch, total_new, chunks, bs_log2);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rotary embedding fused with the packed-QKV unpack and the cache scatter
// (the preprocessing of the same PR, Implementation step 1: rotary,
// packed-QKV unpack, ReshapeAndCache).  One wave per new token: it finds
// the token's sequence and position (kv_len - n_new + i), rotates the first
// rotary_dim features of every Q and K head in fp32 with the angle tables'
// row for that position, writes Q to q_out and K, V into the token's cache
// slot.  Work unit = one 16-byte chunk (8 features), or for the half-split
// pairing a chunk and its partner rotary_dim / 2 features on.

template <bool BF16>
__device__ __forceinline__ f32x2_t unpack2(uint32_t w) {
    if constexpr (BF16) {
        return f32x2_t{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
    } else {
        return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
    }
}

__device__ __forceinline__ u32x4_t ld_chunk(const uint16_t* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ void st_chunk(uint16_t* p, u32x4_t v) {
    *reinterpret_cast<u32x4_t*>(p) = v;
}

// Half-split pairing: features a_0..a_7 (chunk a) pair with b_0..b_7 (chunk
// b) under angles j .. j+7 (cs, sn point at entry j).
template <bool BF16>
__device__ __forceinline__ void rotate_split(u32x4_t& a, u32x4_t& b, const float* cs,
                                             const float* sn) {
    float c[8], sv[8];
    *reinterpret_cast<f32x4_t*>(c) = *reinterpret_cast<const f32x4_t*>(cs);
    *reinterpret_cast<f32x4_t*>(c + 4) = *reinterpret_cast<const f32x4_t*>(cs + 4);
    *reinterpret_cast<f32x4_t*>(sv) = *reinterpret_cast<const f32x4_t*>(sn);
    *reinterpret_cast<f32x4_t*>(sv + 4) = *reinterpret_cast<const f32x4_t*>(sn + 4);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const f32x2_t fa = unpack2<BF16>(a[w]), fb = unpack2<BF16>(b[w]);
        const float cx = c[2 * w], cy = c[2 * w + 1], sx = sv[2 * w], sy = sv[2 * w + 1];
        a[w] = pack2<BF16>(fa.x * cx - fb.x * sx, fa.y * cy - fb.y * sy);
        b[w] = pack2<BF16>(fb.x * cx + fa.x * sx, fb.y * cy + fa.y * sy);
    }
}

// Interleaved pairing: the chunk holds pairs (x_2i, x_2i+1), i = 0..3, under
// angles j .. j+3.
template <bool BF16>
__device__ __forceinline__ u32x4_t rotate_interleaved(u32x4_t x, const float* cs, const float* sn) {
    const f32x4_t c = *reinterpret_cast<const f32x4_t*>(cs);
    const f32x4_t s = *reinterpret_cast<const f32x4_t*>(sn);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const f32x2_t f = unpack2<BF16>(x[w]);
        x[w] = pack2<BF16>(f.x * c[w] - f.y * s[w], f.y * c[w] + f.x * s[w]);
    }
    return x;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_rotary_cache(RotaryParams p) {
    const int lane = lane_id();
    const int waves = gridDim.x * 4;
    const int D = p.head_size, R = p.rotary_dim, half = R / 2;
    const int cpr = D / 8;                                        // chunks per head row
    const int U = (R == 0 || p.interleaved) ? cpr : R / 16 + (D - R) / 8;   // units per head
    const int nq = p.q_out != nullptr ? p.num_heads : 0;
    const int n_rot = (nq + p.num_kv_heads) * U;
    const int n_all = n_rot + p.num_kv_heads * cpr;
    const int64_t row = (int64_t)(p.num_heads + 2 * p.num_kv_heads) * D;
    for (int t = blockIdx.x * 4 + wave_id(); t < p.total_new; t += waves) {
        // sequence of token t: last b with cu_new[b] <= t
        int lo = 0, hi = p.batch;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.cu_new[mid] <= t) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int n_new = p.cu_new[b + 1] - p.cu_new[b];
        const int kv_len = p.cu_kv[b + 1] - p.cu_kv[b];
        const int pos = kv_len - n_new + (t - p.cu_new[b]);
        const int64_t page = p.block_table[(int64_t)b * p.mbps + (pos >> p.bs_log2)];
        const int64_t slot = (page << p.bs_log2) + (pos & ((1 << p.bs_log2) - 1));
        // a position past the tables is a caller error; stay inside them
        const int64_t arow = (int64_t)min(max(pos, 0), max(p.max_position - 1, 0)) * half;
        const float* cs = p.cos + arow;
        const float* sn = p.sin + arow;
        const uint16_t* qs = p.qkv ? p.qkv + t * row : p.q + (int64_t)t * p.num_heads * D;
        const uint16_t* ks = p.qkv ? p.qkv + t * row + p.num_heads * D
                                   : p.k + (int64_t)t * p.num_kv_heads * D;
        const uint16_t* vs = p.qkv ? p.qkv + t * row + (p.num_heads + p.num_kv_heads) * D
                                   : p.v + (int64_t)t * p.num_kv_heads * D;
        for (int u = lane; u < n_all; u += 64) {
            if (u < n_rot) {
                const int hh = u / U, i = u - hh * U;
                const bool isq = hh < nq;
                const uint16_t* src = isq ? qs + hh * D : ks + (hh - nq) * D;
                uint16_t* dst = isq ? p.q_out + ((int64_t)t * p.num_heads + hh) * D
                                    : p.k_cache + (slot * p.num_kv_heads + (hh - nq)) * D;
                if (R == 0) {
                    st_chunk(dst + 8 * i, ld_chunk(src + 8 * i));
                } else if (p.interleaved) {
                    u32x4_t x = ld_chunk(src + 8 * i);
                    if (8 * i < R) x = rotate_interleaved<BF16>(x, cs + 4 * i, sn + 4 * i);
                    st_chunk(dst + 8 * i, x);
                } else if (i < R / 16) {
                    u32x4_t a = ld_chunk(src + 8 * i), bb = ld_chunk(src + half + 8 * i);
                    rotate_split<BF16>(a, bb, cs + 8 * i, sn + 8 * i);
                    st_chunk(dst + 8 * i, a);
                    st_chunk(dst + half + 8 * i, bb);
                } else {
                    const int c = R / 8 + (i - R / 16);
                    st_chunk(dst + 8 * c, ld_chunk(src + 8 * c));
                }
            } else {
                const int vu = u - n_rot, hk = vu / cpr, c = vu - hk * cpr;
                st_chunk(p.v_cache + (slot * p.num_kv_heads + hk) * D + 8 * c,
                         ld_chunk(vs + hk * D + 8 * c));
            }
        }
    }
}

hipError_t launch_rotary_cache(const RotaryParams& p, bool bf16, hipStream_t s) {
    int blocks = (p.total_new + 3) / 4;
    if (blocks > 8192) blocks = 8192;
    if (bf16)
        hipLaunchKernelGGL(k_rotary_cache<true>, dim3(blocks), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(k_rotary_cache<false>, dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace attn
