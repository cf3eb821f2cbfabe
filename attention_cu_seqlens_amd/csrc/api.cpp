// C ABI of the attention library: host-side argument checks, a cached gfx950
// device check and launch planning.  No entry point allocates, frees,
// synchronises or copies device memory to the host.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/attn_cu_seqlens.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
// Longest decode tile list accepted (keeps the split kernel's tile
// positions, and a workgroup's share past them, within int).
constexpr int64_t kDecodeMaxTiles = int64_t{1} << 30;
std::atomic<int> g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

attn_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known == 1) return ATTN_OK;
        if (known == 2) return ATTN_ERR_UNSUPPORTED;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// Tensor base addresses must be 16-byte aligned: the kernels move 16-byte
// chunks.
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// Largest power of two dividing g, at most 8: how many query heads of one
// GQA group share a workgroup's rows.
int pack_log2_for_group(int g) {
    int r = 0;
    while (r < 3 && (g % (2 << r)) == 0) ++r;
    return r;
}

// Local window and score cap: W >= 0, c >= 0 and finite (0 = off).
bool window_cap_ok(int32_t window_left, float softcap) {
    return window_left >= 0 && std::isfinite(softcap) && softcap >= 0.f;
}

// Score-cap constants in the kernels' log2 domain (see SoftCap).
void set_cap(float scale, float softcap, float& in2, float& out) {
    constexpr float kLog2e = 1.4426950408889634f;
    if (softcap > 0.f) {
        in2 = 2.f * std::fabs(scale) * kLog2e / softcap;
        out = softcap * kLog2e;
    } else {
        in2 = 0.f;
        out = 0.f;
    }
}

attn_status check_mask(uint32_t mask, const int32_t* q_ids, const int32_t* kv_ids) {
    if (mask & ~(ATTN_MASK_CAUSAL | ATTN_MASK_DOCUMENT | ATTN_MASK_PATCH))
        return ATTN_ERR_UNSUPPORTED;
    if ((mask & ATTN_MASK_DOCUMENT) && (mask & ATTN_MASK_PATCH)) return ATTN_ERR_UNSUPPORTED;
    if ((mask & ATTN_MASK_DOCUMENT) && (q_ids == nullptr || kv_ids == nullptr))
        return ATTN_ERR_NULL_ARG;
    if ((mask & ATTN_MASK_PATCH) && q_ids == nullptr) return ATTN_ERR_NULL_ARG;
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_string(attn_status status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL_ARG: return "a required pointer is NULL";
        case ATTN_ERR_BAD_SHAPE: return "sizes are inconsistent or out of range";
        case ATTN_ERR_UNSUPPORTED: return "unsupported dtype, head size, mask or device";
        case ATTN_ERR_DEVICE: return "HIP could not report the current device";
        case ATTN_ERR_LAUNCH: return "kernel launch failed";
        case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

attn_status attn_cu_seqlens(const int32_t* seqlens, int32_t* cu_seqlens, int32_t batch,
                            void* stream) {
    if (batch < 0) return ATTN_ERR_BAD_SHAPE;
    if (seqlens == nullptr || cu_seqlens == nullptr) return ATTN_ERR_NULL_ARG;
    if (batch == 0) return ATTN_OK;
    const attn_status d = check_device();
    if (d != ATTN_OK) return d;
    return from_hip(attn::launch_cu_seqlens(seqlens, cu_seqlens, batch,
                                            static_cast<hipStream_t>(stream)));
}

attn_status attn_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* cu_seqlens_new, const int32_t* cu_seqlens_kv,
                                   int32_t batch, int32_t total_new, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t num_blocks,
                                   attn_dtype dtype, void* stream) {
    int esize;
    switch (dtype) {
        case ATTN_F16:
        case ATTN_BF16: esize = 2; break;
        case ATTN_FP8_E4M3: esize = 1; break;
        default: return ATTN_ERR_UNSUPPORTED;
    }
    if (batch < 0 || total_new < 0) return ATTN_ERR_BAD_SHAPE;
    if (num_kv_heads <= 0 || head_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
        return ATTN_ERR_BAD_SHAPE;
    if (!is_pow2(block_size)) return ATTN_ERR_BAD_SHAPE;
    const int64_t row_bytes = (int64_t)num_kv_heads * head_size * esize;
    if (row_bytes % 16 != 0 || row_bytes > (1 << 24)) return ATTN_ERR_BAD_SHAPE;
    if (k == nullptr || v == nullptr || k_cache == nullptr || v_cache == nullptr ||
        block_table == nullptr || cu_seqlens_new == nullptr || cu_seqlens_kv == nullptr)
        return ATTN_ERR_NULL_ARG;
    if (!al16(k) || !al16(v) || !al16(k_cache) || !al16(v_cache)) return ATTN_ERR_BAD_SHAPE;
    if (batch == 0 || total_new == 0) return ATTN_OK;
    const attn_status d = check_device();
    if (d != ATTN_OK) return d;
    return from_hip(attn::launch_reshape_and_cache(
        k, v, k_cache, v_cache, block_table, max_blocks_per_seq, cu_seqlens_new, cu_seqlens_kv,
        batch, total_new, (int)row_bytes, ilog2(block_size), static_cast<hipStream_t>(stream)));
}

attn_status attn_rotary_reshape_and_cache(
    const void* qkv, const void* q, const void* k, const void* v, const float* cos_table,
    const float* sin_table, int32_t max_position, int32_t rotary_dim, int32_t interleaved,
    void* q_out, void* k_cache, void* v_cache, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_new, const int32_t* cu_seqlens_kv,
    int32_t batch, int32_t total_new, int32_t max_seqlen_kv, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t num_blocks,
    attn_dtype dtype, void* stream) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (batch < 0 || total_new < 0 || max_seqlen_kv < 0) return ATTN_ERR_BAD_SHAPE;
    if (num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || head_size % 8 != 0 ||
        head_size > 4096 || num_heads > 4096 || num_kv_heads > 4096)
        return ATTN_ERR_BAD_SHAPE;
    if (max_blocks_per_seq <= 0 || num_blocks <= 0 || !is_pow2(block_size))
        return ATTN_ERR_BAD_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size < max_seqlen_kv) return ATTN_ERR_BAD_SHAPE;
    if (rotary_dim < 0 || rotary_dim % 16 != 0 || rotary_dim > head_size) return ATTN_ERR_BAD_SHAPE;
    if (interleaved != 0 && interleaved != 1) return ATTN_ERR_BAD_SHAPE;
    if (rotary_dim > 0) {
        if (cos_table == nullptr || sin_table == nullptr) return ATTN_ERR_NULL_ARG;
        if (max_position < max_seqlen_kv || max_position <= 0) return ATTN_ERR_BAD_SHAPE;
        if (!al16(cos_table) || !al16(sin_table)) return ATTN_ERR_BAD_SHAPE;
    }
    if (qkv == nullptr && (k == nullptr || v == nullptr || (q_out != nullptr && q == nullptr)))
        return ATTN_ERR_NULL_ARG;
    if (k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
        cu_seqlens_new == nullptr || cu_seqlens_kv == nullptr)
        return ATTN_ERR_NULL_ARG;
    for (const void* ptr : {qkv, q, k, v, static_cast<const void*>(q_out),
                            static_cast<const void*>(k_cache), static_cast<const void*>(v_cache)})
        if (ptr != nullptr && !al16(ptr)) return ATTN_ERR_BAD_SHAPE;
    if (batch == 0 || total_new == 0) return ATTN_OK;
    const attn_status d = check_device();
    if (d != ATTN_OK) return d;
    attn::RotaryParams p{};
    p.qkv = static_cast<const uint16_t*>(qkv);
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.cos = cos_table;
    p.sin = sin_table;
    p.q_out = static_cast<uint16_t*>(q_out);
    p.k_cache = static_cast<uint16_t*>(k_cache);
    p.v_cache = static_cast<uint16_t*>(v_cache);
    p.block_table = block_table;
    p.cu_new = cu_seqlens_new;
    p.cu_kv = cu_seqlens_kv;
    p.mbps = max_blocks_per_seq;
    p.batch = batch;
    p.total_new = total_new;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_size = head_size;
    p.bs_log2 = ilog2(block_size);
    p.rotary_dim = rotary_dim;
    p.max_position = max_position;
    p.interleaved = interleaved;
    return from_hip(attn::launch_rotary_cache(p, dtype == ATTN_BF16, static_cast<hipStream_t>(stream)));
}

size_t attn_varlen_bwd_workspace_bytes(int32_t total_q, int32_t num_heads) {
    if (total_q < 0 || num_heads <= 0) return 0;
    const size_t b = (size_t)total_q * (size_t)num_heads * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

attn_status attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_kv, int32_t batch, int32_t total_q,
                            int32_t total_kv, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            float scale, uint32_t mask_flags, const int32_t* q_ids,
                            const int32_t* kv_ids, int32_t window_left, float softcap,
                            attn_dtype dtype, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (head_size != 64 && head_size != 128) return ATTN_ERR_UNSUPPORTED;
    if (batch < 0 || total_q < 0 || total_kv < 0 || max_seqlen_q < 0 || max_seqlen_kv < 0)
        return ATTN_ERR_BAD_SHAPE;
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
        return ATTN_ERR_BAD_SHAPE;
    if (!std::isfinite(scale) || !window_cap_ok(window_left, softcap)) return ATTN_ERR_BAD_SHAPE;
    const attn_status m = check_mask(mask_flags, q_ids, kv_ids);
    if (m != ATTN_OK) return m;
    // Query-side tensors are required when there are query rows, key-side
    // ones when there are keys (an empty tensor may come as NULL).
    if (cu_seqlens_q == nullptr || cu_seqlens_kv == nullptr ||
        (total_q > 0 && (q == nullptr || out == nullptr || dout == nullptr || lse == nullptr ||
                         dq == nullptr)) ||
        (total_kv > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)))
        return ATTN_ERR_NULL_ARG;
    for (const void* ptr : {q, k, v, out, dout, static_cast<const void*>(dq),
                            static_cast<const void*>(dk), static_cast<const void*>(dv)})
        if (!al16(ptr)) return ATTN_ERR_BAD_SHAPE;
    if (batch == 0 || (total_q == 0 && total_kv == 0)) return ATTN_OK;
    const size_t need = attn_varlen_bwd_workspace_bytes(total_q, num_heads);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                     ((uintptr_t)workspace & 255) != 0))
        return ATTN_ERR_WORKSPACE;
    const attn_status d = check_device();
    if (d != ATTN_OK) return d;
    attn::BwdParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.out = static_cast<const uint16_t*>(out);
    p.dout = static_cast<const uint16_t*>(dout);
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_kv = cu_seqlens_kv;
    p.q_ids = q_ids;
    p.kv_ids = kv_ids;
    p.dq = static_cast<uint16_t*>(dq);
    p.dk = static_cast<uint16_t*>(dk);
    p.dv = static_cast<uint16_t*>(dv);
    p.delta = static_cast<float*>(workspace);
    p.batch = batch;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_heads / num_kv_heads;
    p.total_q = total_q;
    p.mask = mask_flags;
    p.window = window_left;
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    if (softcap > 0.f) {
        p.cap_in2 = 2.f * 1.4426950408889634f * scale / softcap;
        p.cap_out = softcap * 1.4426950408889634f;
    }
    return from_hip(attn::launch_varlen_bwd(p, head_size, dtype == ATTN_BF16, max_seqlen_q,
                                            max_seqlen_kv, static_cast<hipStream_t>(stream)));
}

namespace {

// Stored block-sparse mask arguments (null kv_num: none).
struct BlockSparseArgs {
    int32_t q_block, kv_block, mask_heads, num_q_blocks, capacity;
    const int32_t* kv_num;
    const int32_t* kv_idx;
    const int32_t* full_num;
    const int32_t* full_idx;
};

attn_status prefill_impl(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int32_t batch,
                         int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int32_t num_blocks, float scale, uint32_t mask_flags,
                         const int32_t* q_ids, const int32_t* kv_ids, int32_t window_left,
                         float softcap, const BlockSparseArgs* bm, attn_dtype dtype, void* out,
                         float* lse, void* stream) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (head_size != 64 && head_size != 128) return ATTN_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32 && block_size != 64) return ATTN_ERR_UNSUPPORTED;
    if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_kv < 0)
        return ATTN_ERR_BAD_SHAPE;
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
        return ATTN_ERR_BAD_SHAPE;
    if (max_blocks_per_seq <= 0 || num_blocks <= 0) return ATTN_ERR_BAD_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size < max_seqlen_kv) return ATTN_ERR_BAD_SHAPE;
    if (!std::isfinite(scale)) return ATTN_ERR_BAD_SHAPE;
    if (!window_cap_ok(window_left, softcap)) return ATTN_ERR_BAD_SHAPE;
    const attn_status m = check_mask(mask_flags, q_ids, kv_ids);
    if (m != ATTN_OK) return m;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
        cu_seqlens_q == nullptr || cu_seqlens_kv == nullptr || out == nullptr)
        return ATTN_ERR_NULL_ARG;
    if (!al16(q) || !al16(k_cache) || !al16(v_cache) || !al16(out)) return ATTN_ERR_BAD_SHAPE;
    const int group = num_heads / num_kv_heads;
    // a mask with one list per query head needs one head per workgroup
    int pack_log2 = pack_log2_for_group(group);
    int n_kb = 0;
    if (bm != nullptr) {
        if (bm->kv_num == nullptr || bm->kv_idx == nullptr) return ATTN_ERR_NULL_ARG;
        if ((bm->full_num == nullptr) != (bm->full_idx == nullptr)) return ATTN_ERR_NULL_ARG;
        if (!is_pow2(bm->q_block) || bm->q_block < 32 || bm->q_block > (1 << 30) ||
            !is_pow2(bm->kv_block) || bm->kv_block < 64 || bm->kv_block > (1 << 30))
            return ATTN_ERR_UNSUPPORTED;
        if (bm->mask_heads != 1 && bm->mask_heads != num_kv_heads && bm->mask_heads != num_heads)
            return ATTN_ERR_BAD_SHAPE;
        if (bm->capacity <= 0 || bm->num_q_blocks <= 0 ||
            (int64_t)bm->num_q_blocks * bm->q_block < max_seqlen_q)
            return ATTN_ERR_BAD_SHAPE;
        if (bm->mask_heads == num_heads && num_heads != num_kv_heads) pack_log2 = 0;
        n_kb = (int)std::max<int64_t>(1, ((int64_t)max_seqlen_kv + bm->kv_block - 1) / bm->kv_block);
        const int n_lq = std::max(1, (attn::kPrefillRows >> pack_log2) / bm->q_block);
        if ((int64_t)n_lq * n_kb > attn::kBlockStateBytes) return ATTN_ERR_UNSUPPORTED;
    }
    if (batch == 0 || total_q == 0) return ATTN_OK;
    const attn_status d = check_device();
    if (d != ATTN_OK) return d;

    attn::PrefillParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k_cache = static_cast<const uint16_t*>(k_cache);
    p.v_cache = static_cast<const uint16_t*>(v_cache);
    p.block_table = block_table;
    p.cu_q = cu_seqlens_q;
    p.cu_kv = cu_seqlens_kv;
    p.q_ids = q_ids;
    p.kv_ids = kv_ids;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.mbps = max_blocks_per_seq;
    p.batch = batch;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = group;
    p.pack_log2 = pack_log2;
    p.n_head_groups = num_heads >> p.pack_log2;
    p.total_q = total_q;
    p.bs_log2 = ilog2(block_size);
    p.mask = mask_flags;
    p.c = scale * 1.4426950408889634f;
    p.window = window_left;
    set_cap(scale, softcap, p.cap_in2, p.cap_out);
    if (bm != nullptr) {
        p.bm_kv_num = bm->kv_num;
        p.bm_kv_idx = bm->kv_idx;
        p.bm_full_num = bm->full_num;
        p.bm_full_idx = bm->full_idx;
        p.bm_heads = bm->mask_heads;
        p.bm_nqb = bm->num_q_blocks;
        p.bm_cap = bm->capacity;
        p.bm_n_kb = n_kb;
        p.bm_qbs_log2 = ilog2(bm->q_block);
        p.bm_kvbs_log2 = ilog2(bm->kv_block);
    }
    return from_hip(attn::launch_paged_prefill(p, head_size, dtype == ATTN_BF16, max_seqlen_q,
                                               static_cast<hipStream_t>(stream)));
}

}  // namespace

attn_status attn_paged_prefill_fwd(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                   int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                   int32_t max_seqlen_kv, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t num_blocks,
                                   float scale, uint32_t mask_flags, const int32_t* q_ids,
                                   const int32_t* kv_ids, int32_t window_left, float softcap,
                                   attn_dtype dtype, void* out, float* lse, void* stream) {
    return prefill_impl(q, k_cache, v_cache, block_table, max_blocks_per_seq, cu_seqlens_q,
                        cu_seqlens_kv, batch, total_q, max_seqlen_q, max_seqlen_kv, num_heads,
                        num_kv_heads, head_size, block_size, num_blocks, scale, mask_flags, q_ids,
                        kv_ids, window_left, softcap, nullptr, dtype, out, lse, stream);
}

attn_status attn_paged_prefill_block_sparse_fwd(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, uint32_t mask_flags, const int32_t* q_ids,
    const int32_t* kv_ids, int32_t window_left, float softcap, int32_t q_block, int32_t kv_block,
    int32_t mask_heads, int32_t num_q_blocks, int32_t list_capacity,
    const int32_t* kv_num_blocks, const int32_t* kv_indices, const int32_t* full_kv_num_blocks,
    const int32_t* full_kv_indices, attn_dtype dtype, void* out, float* lse, void* stream) {
    const BlockSparseArgs bm{q_block, kv_block, mask_heads, num_q_blocks, list_capacity,
                             kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices};
    return prefill_impl(q, k_cache, v_cache, block_table, max_blocks_per_seq, cu_seqlens_q,
                        cu_seqlens_kv, batch, total_q, max_seqlen_q, max_seqlen_kv, num_heads,
                        num_kv_heads, head_size, block_size, num_blocks, scale, mask_flags, q_ids,
                        kv_ids, window_left, softcap, &bm, dtype, out, lse, stream);
}

size_t attn_paged_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_size, int32_t max_seqlen_kv,
                                         int32_t window_left, int32_t split_tokens) {
    if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 || max_seqlen_kv < 0)
        return 0;
    if (split_tokens < 0 || split_tokens % 256 != 0 || split_tokens > 8192) return 0;
    if (window_left < 0) return 0;
    if (attn::decode_tile_bound(batch, num_kv_heads, max_seqlen_kv, window_left) > kDecodeMaxTiles)
        return 0;
    return attn::decode_workspace(batch, num_heads, num_kv_heads, head_size, max_seqlen_kv,
                                  window_left, split_tokens)
        .bytes;
}

}  // extern "C"

namespace {

// Decode over a 16-bit cache (kv_descale == nullptr) or an fp8 e4m3 cache.
attn_status decode_impl(const void* q, const void* k_cache, const void* v_cache, bool kv8,
                        const float* kv_descale, const int32_t* block_table,
                        int32_t max_blocks_per_seq, const int32_t* cu_seqlens_kv, int32_t batch,
                        int32_t max_seqlen_kv, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_size, int32_t block_size, int32_t num_blocks, float scale,
                        int32_t window_left, float softcap, int32_t split_tokens, attn_dtype dtype,
                        void* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream, bool use_scratch = false) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (head_size != 64 && head_size != 128) return ATTN_ERR_UNSUPPORTED;
    if (block_size != 16 && block_size != 32 && block_size != 64) return ATTN_ERR_UNSUPPORTED;
    if (batch < 0 || max_seqlen_kv < 0) return ATTN_ERR_BAD_SHAPE;
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
        return ATTN_ERR_BAD_SHAPE;
    if (num_heads / num_kv_heads > 32) return ATTN_ERR_UNSUPPORTED;
    if (max_blocks_per_seq <= 0 || num_blocks <= 0) return ATTN_ERR_BAD_SHAPE;
    if ((int64_t)max_blocks_per_seq * block_size < max_seqlen_kv) return ATTN_ERR_BAD_SHAPE;
    if (split_tokens < 0 || split_tokens % 256 != 0 || split_tokens > 8192)
        return ATTN_ERR_BAD_SHAPE;
    if (!std::isfinite(scale)) return ATTN_ERR_BAD_SHAPE;
    if (!window_cap_ok(window_left, softcap)) return ATTN_ERR_BAD_SHAPE;
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
        cu_seqlens_kv == nullptr || out == nullptr || (kv8 && kv_descale == nullptr))
        return ATTN_ERR_NULL_ARG;
    if (!al16(q) || !al16(k_cache) || !al16(v_cache) || !al16(out)) return ATTN_ERR_BAD_SHAPE;
    if (batch == 0) return ATTN_OK;
    if (attn::decode_tile_bound(batch, num_kv_heads, max_seqlen_kv, window_left) > kDecodeMaxTiles)
        return ATTN_ERR_BAD_SHAPE;
    const attn::DecodeWorkspace lay = attn::decode_workspace(
        batch, num_heads, num_kv_heads, head_size, max_seqlen_kv, window_left, split_tokens);
    const size_t need = lay.bytes;
    if (use_scratch) {
        // the library's own scratch array (no allocation): size checked here,
        // on the host, before any HIP call
        if (need > attn::kDecodeScratchBytes) return ATTN_ERR_WORKSPACE;
    } else if (workspace == nullptr || workspace_bytes < need ||
               (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) {
        return ATTN_ERR_WORKSPACE;
    }
    const attn_status d = check_device();
    if (d != ATTN_OK) return d;
    if (use_scratch) {
        if (attn::decode_scratch(&workspace) != hipSuccess) return ATTN_ERR_DEVICE;
        workspace_bytes = attn::kDecodeScratchBytes;
    }

    attn::DecodeParams p{};
    p.q = static_cast<const uint16_t*>(q);
    if (kv8) {
        p.k8 = static_cast<const uint8_t*>(k_cache);
        p.v8 = static_cast<const uint8_t*>(v_cache);
        p.kv_descale = kv_descale;
    } else {
        p.k_cache = static_cast<const uint16_t*>(k_cache);
        p.v_cache = static_cast<const uint16_t*>(v_cache);
    }
    p.block_table = block_table;
    p.cu_kv = cu_seqlens_kv;
    int cus = 0;
    if (attn::cu_count(&cus) != hipSuccess) return ATTN_ERR_DEVICE;
    p.grid = attn::decode_grid(batch, num_kv_heads, max_seqlen_kv, window_left, split_tokens,
                               2 * cus);
    p.split_tiles = split_tokens / 32;
    p.part_o = static_cast<float*>(workspace);
    p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.ml_off);
    p.seg_meta = reinterpret_cast<int*>(static_cast<char*>(workspace) + lay.meta_off);
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    p.mbps = max_blocks_per_seq;
    p.batch = batch;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_heads / num_kv_heads;
    p.head_pack = attn::decode_head_pack(num_kv_heads);
    p.bs_log2 = ilog2(block_size);
    p.c = scale * 1.4426950408889634f;
    p.window = window_left;
    set_cap(scale, softcap, p.cap_in2, p.cap_out);
    return from_hip(attn::launch_paged_decode(p, head_size, dtype == ATTN_BF16,
                                              static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

attn_status attn_paged_decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* cu_seqlens_kv, int32_t batch,
                                  int32_t max_seqlen_kv, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t block_size, int32_t num_blocks,
                                  float scale, int32_t window_left, float softcap,
                                  int32_t split_tokens, attn_dtype dtype, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(q, k_cache, v_cache, false, nullptr, block_table, max_blocks_per_seq,
                       cu_seqlens_kv, batch, max_seqlen_kv, num_heads, num_kv_heads, head_size,
                       block_size, num_blocks, scale, window_left, softcap, split_tokens, dtype,
                       out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_paged_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* cu_seqlens_kv, int32_t batch,
                                          int32_t max_seqlen_kv, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_size,
                                          int32_t block_size, int32_t num_blocks, float scale,
                                          int32_t window_left, float softcap,
                                          int32_t split_tokens, attn_dtype dtype, void* out,
                                          float* lse, void* stream) {
    static_assert(ATTN_DECODE_SCRATCH_BYTES == attn::kDecodeScratchBytes, "scratch size");
    return decode_impl(q, k_cache, v_cache, false, nullptr, block_table, max_blocks_per_seq,
                       cu_seqlens_kv, batch, max_seqlen_kv, num_heads, num_kv_heads, head_size,
                       block_size, num_blocks, scale, window_left, softcap, split_tokens, dtype,
                       out, lse, nullptr, 0, stream, /*use_scratch=*/true);
}

attn_status attn_paged_decode_fp8kv_fwd(const void* q, const void* k_cache8, const void* v_cache8,
                                        const float* kv_descale, const int32_t* block_table,
                                        int32_t max_blocks_per_seq, const int32_t* cu_seqlens_kv,
                                        int32_t batch, int32_t max_seqlen_kv, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t block_size, int32_t num_blocks, float scale,
                                        int32_t window_left, float softcap, int32_t split_tokens,
                                        attn_dtype q_dtype, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    return decode_impl(q, k_cache8, v_cache8, true, kv_descale, block_table, max_blocks_per_seq,
                       cu_seqlens_kv, batch, max_seqlen_kv, num_heads, num_kv_heads, head_size,
                       block_size, num_blocks, scale, window_left, softcap, split_tokens, q_dtype,
                       out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_fp8_fwd(const void* q8, const void* k8, const void* v8_colmajor,
                         const float* descale_qkv, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_kv, int32_t batch, int32_t total_q,
                         int32_t total_kv, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_size, float scale,
                         uint32_t mask_flags, const int32_t* q_ids, const int32_t* kv_ids,
                         int32_t window_left, float softcap, void* out_bf16, float* lse,
                         void* stream) {
    if (head_size != 128) return ATTN_ERR_UNSUPPORTED;
    if (batch < 0 || total_q < 0 || total_kv < 0 || max_seqlen_q < 0 || max_seqlen_kv < 0)
        return ATTN_ERR_BAD_SHAPE;
    if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0)
        return ATTN_ERR_BAD_SHAPE;
    if (!std::isfinite(scale)) return ATTN_ERR_BAD_SHAPE;
    if (!window_cap_ok(window_left, softcap)) return ATTN_ERR_BAD_SHAPE;
    const attn_status m = check_mask(mask_flags, q_ids, kv_ids);
    if (m != ATTN_OK) return m;
    if (q8 == nullptr || k8 == nullptr || v8_colmajor == nullptr || descale_qkv == nullptr ||
        cu_seqlens_q == nullptr || cu_seqlens_kv == nullptr || out_bf16 == nullptr)
        return ATTN_ERR_NULL_ARG;
    if (!al16(q8) || !al16(k8) || !al16(v8_colmajor) || !al16(out_bf16))
        return ATTN_ERR_BAD_SHAPE;
    // the kernel addresses 32 V rows of one head with 32-bit offsets
    if (total_kv > (1 << 27)) return ATTN_ERR_BAD_SHAPE;
    if (batch == 0 || total_q == 0) return ATTN_OK;
    const attn_status d = check_device();
    if (d != ATTN_OK) return d;

    attn::Fp8Params p{};
    p.q = static_cast<const uint8_t*>(q8);
    p.k = static_cast<const uint8_t*>(k8);
    p.vt = static_cast<const uint8_t*>(v8_colmajor);
    p.descale = descale_qkv;
    p.cu_q = cu_seqlens_q;
    p.cu_kv = cu_seqlens_kv;
    p.q_ids = q_ids;
    p.kv_ids = kv_ids;
    p.out = static_cast<uint16_t*>(out_bf16);
    p.lse = lse;
    p.batch = batch;
    p.total_kv = total_kv;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = num_heads / num_kv_heads;
    p.pack_log2 = pack_log2_for_group(p.group);
    p.n_head_groups = num_heads >> p.pack_log2;
    p.total_q = total_q;
    p.mask = mask_flags;
    p.scale = scale;
    p.window = window_left;
    p.softcap = softcap;
    return from_hip(attn::launch_fp8_prefill(p, head_size, max_seqlen_q,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
