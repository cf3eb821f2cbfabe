// Kernel parameter blocks and launchers (internal; the public ABI is
// include/attn_cu_seqlens.h).  Launchers return a hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

enum : uint32_t { kMaskCausal = 1u, kMaskDocument = 2u, kMaskPatch = 4u };

// Paged varlen prefill (16-bit dtypes).
struct PrefillParams {
    const uint16_t* q;          // [total_q, Hq, D]
    const uint16_t* k_cache;    // [num_blocks, bs, Hkv, D]
    const uint16_t* v_cache;
    const int32_t* block_table; // [batch, mbps]
    const int32_t* cu_q;
    const int32_t* cu_kv;
    const int32_t* q_ids;
    const int32_t* kv_ids;
    uint16_t* out;              // [total_q, Hq, D]
    float* lse;                 // [total_q, Hq] or null
    int mbps;
    int batch;
    int num_heads;
    int num_kv_heads;
    int group;                  // num_heads / num_kv_heads
    int pack_log2;              // log2 of q heads packed per workgroup
    int n_head_groups;          // num_heads >> pack_log2
    int n_qtiles;               // tiles per sequence at max_seqlen_q
    int total_q;
    int bs_log2;
    uint32_t mask;
    float c;                    // scale * log2(e)
    int window;                 // local window (keys), 0 = none
    float cap_in2, cap_out;     // score cap constants (SoftCap), cap_out == 0: none
    // stored block-sparse mask (bm_kv_num null: none).  Lists per (sequence,
    // mask head, query block): [batch, bm_heads, bm_nqb] counts and
    // [batch, bm_heads, bm_nqb, bm_cap] kv-block ids; the full pair may be null.
    const int32_t* bm_kv_num;
    const int32_t* bm_kv_idx;
    const int32_t* bm_full_num;
    const int32_t* bm_full_idx;
    int bm_heads;               // 1, num_kv_heads or num_heads
    int bm_nqb;                 // query blocks per sequence in the arrays
    int bm_cap;                 // list capacity
    int bm_n_kb;                // ceil(max_seqlen_kv / kv block): state row length
    int bm_qbs_log2, bm_kvbs_log2;
    int wg_per_xcd;             // persistent launch: workgroups per XCD
};

// Rotary + packed-QKV unpack + reshape_and_cache, one pass over the new
// tokens (16-bit dtypes).
struct RotaryParams {
    const uint16_t* qkv;        // packed [total_new, (Hq + 2 Hkv) * D] or null
    const uint16_t* q;          // separate inputs (qkv null): [total_new, Hq, D]
    const uint16_t* k;          // [total_new, Hkv, D]
    const uint16_t* v;
    const float* cos;           // [max_position, rotary_dim / 2]
    const float* sin;
    uint16_t* q_out;            // [total_new, Hq, D] or null (Q not written)
    uint16_t* k_cache;          // [num_blocks, bs, Hkv, D]
    uint16_t* v_cache;
    const int32_t* block_table;
    const int32_t* cu_new;
    const int32_t* cu_kv;
    int mbps, batch, total_new, num_heads, num_kv_heads, head_size, bs_log2;
    int rotary_dim;             // 0: no rotation
    int max_position;
    int interleaved;
};

// Varlen backward (16-bit dtypes, packed K/V): delta, dQ and dK/dV kernels.
struct BwdParams {
    const uint16_t* q;          // [total_q, Hq, D]
    const uint16_t* k;          // [total_kv, Hkv, D]
    const uint16_t* v;
    const uint16_t* out;        // forward output [total_q, Hq, D]
    const uint16_t* dout;       // upstream gradient [total_q, Hq, D]
    const float* lse;           // [total_q, Hq], natural log
    const int32_t* cu_q;
    const int32_t* cu_kv;
    const int32_t* q_ids;
    const int32_t* kv_ids;
    uint16_t* dq;               // [total_q, Hq, D]
    uint16_t* dk;               // [total_kv, Hkv, D]
    uint16_t* dv;
    float* delta;               // workspace [total_q, Hq]: rowsum(dO * O)
    int batch, num_heads, num_kv_heads, group, total_q;
    uint32_t mask;
    int window;
    float scale;
    float c;                    // scale * log2(e)
    float cap_in2;              // score cap: 2 log2(e) scale / cap (signed)
    float cap_out;              // cap * log2(e); 0: no cap
    int n_qt, n_kt;             // 128-row query / key tiles per sequence at the max lengths
};

// Query rows (token x packed head) per prefill workgroup, and the bytes of
// its block-sparse state: one byte per (local query block, key block).
constexpr int kPrefillRows = 256;
constexpr int kBlockStateBytes = 16384;

// Paged decode (16-bit dtypes): split kernel + combine kernel.
struct DecodeParams {
    const uint16_t* q;          // [batch, Hq, D]
    const uint16_t* k_cache;    // 16-bit cache (null when k8 is set)
    const uint16_t* v_cache;
    const uint8_t* k8;          // fp8 e4m3 cache (same layout, bytes) or null
    const uint8_t* v8;
    const float* kv_descale;    // [2] device (dk, dv) with k8
    const int32_t* block_table;
    const int32_t* cu_kv;
    float* part_o;              // [slots, HP*G, D] segment partials (slot = unit + workgroup)
    float* part_ml;             // [slots, HP*G, 2] their running max and sum
    int* seg_meta;              // [batch*Hkv/HP, 2] first slot and segment count per unit
    uint16_t* out;              // [batch, Hq, D]
    float* lse;                 // [batch, Hq] or null
    int mbps;
    int batch;
    int num_heads;
    int num_kv_heads;
    int group;
    int head_pack;              // HP: kv heads per unit (decode_head_pack)
    int bs_log2;
    int split_tiles;            // tiles per workgroup, 0: balanced over the grid
    int grid;                   // workgroups of the split kernel
    float c;
    int window;                 // local window (keys), 0 = none
    float cap_in2, cap_out;     // score cap constants (SoftCap), cap_out == 0: none
};

// Dense varlen fp8 prefill.
struct Fp8Params {
    const uint8_t* q;           // [total_q, Hq, D]
    const uint8_t* k;           // [total_kv, Hkv, D]
    const uint8_t* vt;          // [Hkv, D, total_kv]
    const float* descale;       // [3] device
    const int32_t* cu_q;
    const int32_t* cu_kv;
    const int32_t* q_ids;
    const int32_t* kv_ids;
    uint16_t* out;              // bf16 [total_q, Hq, D]
    float* lse;
    int batch;
    int total_kv;
    int num_heads;
    int num_kv_heads;
    int group;
    int pack_log2;
    int n_head_groups;
    int n_qtiles;
    int total_q;
    uint32_t mask;
    float scale;
    int window;                 // local window (keys), 0 = none
    float softcap;              // score cap c, 0 = none
};

hipError_t launch_cu_seqlens(const int32_t* seqlens, int32_t* cu, int batch, hipStream_t s);
hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int32_t* block_table, int mbps, const int32_t* cu_new,
                                    const int32_t* cu_kv, int batch, int total_new,
                                    int row_bytes, int bs_log2, hipStream_t s);
hipError_t launch_rotary_cache(const RotaryParams& p, bool bf16, hipStream_t s);
hipError_t launch_varlen_bwd(const BwdParams& p, int head_size, bool bf16, int max_seqlen_q,
                             int max_seqlen_kv, hipStream_t s);
hipError_t launch_paged_prefill(const PrefillParams& p, int head_size, bool bf16,
                                int max_seqlen_q, hipStream_t s);
hipError_t launch_paged_decode(const DecodeParams& p, int head_size, bool bf16, hipStream_t s);
hipError_t launch_fp8_prefill(const Fp8Params& p, int head_size, int max_seqlen_q, hipStream_t s);

// Scratch of the allocation-free decode entry point (one array per GPU).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
// Device address of this GPU's scratch array (the current device), looked up
// once per device.
hipError_t decode_scratch(void** ptr);

// Compute units of the current device (looked up once per device).
hipError_t cu_count(int* out);

// Decode planning shared by the workspace query and the launch.
// Shortest share of the tile list a workgroup takes by default (512 keys),
// and the most workgroups the default grid uses (two per CU up to 512 CUs).
constexpr int kDecodeMinSegTiles = 16;
constexpr int kDecodeMaxGrid = 1024;
int decode_head_pack(int num_kv_heads);
int decode_span(int max_seqlen_kv, int window);
int64_t decode_tile_bound(int batch, int num_kv_heads, int max_seqlen_kv, int window);
int decode_grid(int batch, int num_kv_heads, int max_seqlen_kv, int window, int split_tokens,
                int resident);
struct DecodeWorkspace {
    size_t ml_off, meta_off, bytes;   // byte offsets of part_ml and seg_meta; total size
};
DecodeWorkspace decode_workspace(int batch, int num_heads, int num_kv_heads, int head_size,
                                 int max_seqlen_kv, int window, int split_tokens);

}  // namespace attn
