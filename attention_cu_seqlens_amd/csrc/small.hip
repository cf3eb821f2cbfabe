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

}  // namespace attn
