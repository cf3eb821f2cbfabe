/*
 * attn_cu_seqlens -- varlen, paged, GQA attention forward for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is caller-owned DEVICE memory unless stated
 * otherwise; the library never allocates, frees, synchronises or copies device
 * memory to the host.  Each call enqueues its kernels on `stream` (a
 * hipStream_t; NULL is the default stream) and returns at once.  Argument
 * checks run on the host before any HIP call; a failed check returns an error
 * code and launches nothing.  No function aborts the process.
 *
 * Conventions shared by all entry points
 *   - Packed varlen ("BSNH") tensors: token-major, [total_tokens, heads,
 *     head_size], contiguous.  Sequence b owns tokens cu[b] .. cu[b+1]-1 of a
 *     cumulative-length array cu[batch+1] with cu[0] = 0 (the cumulative
 *     seqlens of the onnxruntime PR "[CUDA] PagedAttention: add SM<80 fp16
 *     fallback via memory-efficient attention", section Implementation,
 *     steps 1 and 3).
 *   - Paged K/V cache: [num_blocks, block_size, num_kv_heads, head_size];
 *     block_table is int32 [batch, max_blocks_per_seq] and maps logical block
 *     i of sequence b to physical block block_table[b*max_blocks_per_seq + i]
 *     (same PR, Implementation step 2 and the size formula under "Scratch
 *     allocation").  Token j of sequence b lives in physical block
 *     block_table[b][j / block_size] at slot j % block_size.  Entries past
 *     ceil(kv_len / block_size) are never read; cache slots past kv_len are
 *     never read into a result (they may hold any bits, NaN included).
 *   - GQA: query head h reads kv head h / (num_heads / num_kv_heads).
 *   - Scores are scale * <q, k> (the scale multiplies the product, not q:
 *     "PRESCALE_QK: False" among the FlexAttention kernel options in the blt
 *     issue "Cross Attention does not work on CPU and older GPUs").  Callers
 *     wanting the usual default pass 1/sqrt(head_size) (flex_attention
 *     docstring in the pytorch commit "[FlexAttention] Enforce Q,K,V memory
 *     layouts for fp8 flex attention to avoid perf degradation").
 *   - Masks (mask_flags): ATTN_MASK_CAUSAL keeps key j for query i iff
 *     j <= i + kv_len - q_len (bottom-right alignment; equals the page's
 *     q_idx >= kv_idx when lengths match).  ATTN_MASK_DOCUMENT keeps j iff
 *     q_ids[q] == kv_ids[k] (document ids, non-decreasing within each
 *     sequence).  ATTN_MASK_PATCH keeps j iff j <= q_ids[q], where q_ids is
 *     each query byte's patch index within its sequence (non-decreasing) --
 *     the byte->patch cross-attention of the blt issue.  CAUSAL combines with
 *     either; DOCUMENT and PATCH are exclusive.  q_ids / kv_ids are indexed by
 *     global token (q_ids[total_q], kv_ids[total_kv]).
 *   - Local window and score cap (window_left, softcap): the onnxruntime PR's
 *     parity matrix runs "local window on/off" and "softcap 0/50" (section
 *     Testing) without defining them; read here as
 *       window_left W > 0: key j is kept only if j > i + kv_len - q_len - W,
 *       a window of W keys ending at the query's own (bottom-right) position,
 *       combined with the mask flags; W = 0 means no window;
 *       softcap c > 0: every scaled score s becomes c * tanh(s / c) before
 *       the mask and the softmax (LSE is over the capped scores); c = 0
 *       means no cap.
 *     Negative, NaN or infinite values are ATTN_ERR_BAD_SHAPE.
 *   - A query row with no visible key outputs zeros and LSE = -inf (rows may
 *     be fully masked: "ROWS_GUARANTEED_SAFE: False" in the same kernel
 *     options).
 *   - lse (optional, may be NULL): float32 [total_q, num_heads], natural-log
 *     logsumexp of the scaled, masked scores ("OUTPUT_LOGSUMEXP: True").
 *   - Accumulation is fp32 whatever the input dtype; outputs are rounded to
 *     nearest even.
 *   - Device-resident metadata (cu_seqlens, block_table, ids) is trusted:
 *     cu arrays must be non-decreasing with cu[batch] equal to the stated
 *     total, used table entries must lie in [0, num_blocks), and no sequence
 *     may be longer than the max_seqlen arguments.
 *   - Tensor arguments (q, k, v, caches, out) must start on a 16-byte
 *     boundary; otherwise ATTN_ERR_BAD_SHAPE.
 *   - The device must be gfx950; otherwise ATTN_ERR_UNSUPPORTED.  The check
 *     runs on the first call on each device and is cached.
 *   - Calls with nothing to compute (batch == 0, total == 0) return ATTN_OK
 *     without touching the GPU.
 */
#ifndef ATTN_CU_SEQLENS_H
#define ATTN_CU_SEQLENS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 4

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
    ATTN_ERR_BAD_SHAPE = 2,    /* sizes inconsistent or out of range */
    ATTN_ERR_UNSUPPORTED = 3,  /* dtype / head_size / mask / device not supported */
    ATTN_ERR_DEVICE = 4,       /* HIP could not report the current device */
    ATTN_ERR_LAUNCH = 5,       /* a kernel launch failed (hipGetLastError) */
    ATTN_ERR_WORKSPACE = 6     /* workspace missing or too small */
} attn_status;

typedef enum attn_dtype {
    ATTN_F16 = 0,
    ATTN_BF16 = 1,
    ATTN_FP8_E4M3 = 2          /* OCP e4m3fn */
} attn_dtype;

#define ATTN_MASK_NONE 0u
#define ATTN_MASK_CAUSAL 1u
#define ATTN_MASK_DOCUMENT 2u
#define ATTN_MASK_PATCH 4u

/* Version of this ABI (ATTN_ABI_VERSION). */
int attn_abi_version(void);

/* Static text for a status code (never NULL). */
const char* attn_status_string(attn_status status);

/*
 * attn_cu_seqlens -- cumulative sequence lengths.
 * The cumulative-seqlens buffer of the onnxruntime PR (section
 * Implementation: LaunchGetCumulativeSeqlensKV, whose element [batch_size]
 * is the token total).
 *   seqlens     int32 [batch], each >= 0 (device)
 *   cu_seqlens  int32 [batch + 1] output (device): cu[0] = 0,
 *               cu[b+1] = cu[b] + seqlens[b].  Must not alias seqlens.
 * The caller guarantees the total fits int32.  batch == 0 writes nothing.
 * Errors: NULL pointer, batch < 0.
 */
attn_status attn_cu_seqlens(const int32_t* seqlens, int32_t* cu_seqlens, int32_t batch,
                            void* stream);

/*
 * attn_reshape_and_cache -- append new K/V tokens to the paged cache.
 * ReshapeAndCache of the onnxruntime PR (section Implementation, step 1).
 * Sequence b appends n = cu_seqlens_new[b+1] - cu_seqlens_new[b] tokens and
 * afterwards holds kv_len = cu_seqlens_kv[b+1] - cu_seqlens_kv[b] tokens
 * (n <= kv_len), so new token i goes to position kv_len - n + i.
 *   k, v              [total_new, num_kv_heads, head_size] (device)
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_size], written
 *   block_table       int32 [batch, max_blocks_per_seq]
 *   dtype             any attn_dtype (the copy is bitwise)
 * Only the addressed slots are written.  Errors: NULL pointer, non-positive
 * sizes, head_size not a multiple of 16 bytes / element size, block_size not
 * a power of two, unsupported dtype.
 */
attn_status attn_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* cu_seqlens_new, const int32_t* cu_seqlens_kv,
                                   int32_t batch, int32_t total_new, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t num_blocks,
                                   attn_dtype dtype, void* stream);

/*
 * attn_rotary_reshape_and_cache -- the rest of the onnxruntime PR's
 * preprocessing (section Implementation, step 1: rotary, packed-QKV unpack,
 * ReshapeAndCache) in one pass over the new tokens: unpack, rotate Q and K,
 * write Q to q_out and K, V into the cache like attn_reshape_and_cache.
 * Rotary: the first rotary_dim features of every Q and K head are rotated in
 * pairs by the angle-table row of the token's position pos = kv_len - n + i
 * (where attn_reshape_and_cache puts it): with c = cos_table[pos][j],
 * s = sin_table[pos][j], a pair (a, b) becomes (a c - b s, b c + a s).
 * interleaved = 0 pairs feature j with j + rotary_dim/2, interleaved = 1
 * pairs 2j with 2j+1 (j < rotary_dim/2).  Features past rotary_dim and V are
 * copied.  Arithmetic in fp32, results rounded to nearest even.
 *   qkv          packed [total_new, (num_heads + 2 * num_kv_heads) * head_size]:
 *                per token the query heads, then the key heads, then the
 *                value heads; or NULL, then q, k, v are read:
 *   q            [total_new, num_heads, head_size] (may be NULL when q_out is)
 *   k, v         [total_new, num_kv_heads, head_size]
 *   cos_table, sin_table  float32 [max_position, rotary_dim / 2] (device),
 *                NULL allowed when rotary_dim == 0; max_position must be at
 *                least max_seqlen_kv (every position is below kv_len)
 *   rotary_dim   0 (no rotation) or a multiple of 16 up to head_size
 *   q_out        [total_new, num_heads, head_size], or NULL to skip Q; may
 *                be q itself (each element is read before it is written)
 *   k_cache, v_cache, block_table, cu_seqlens_new, cu_seqlens_kv  as
 *                attn_reshape_and_cache
 *   dtype        ATTN_F16 or ATTN_BF16 (inputs, q_out and caches)
 * All buffers 16-byte aligned device memory.  Errors: NULL pointer, bad
 * shape (sizes, rotary_dim, max_position, head_size not a multiple of 8,
 * alignment), unsupported dtype.
 */
attn_status attn_rotary_reshape_and_cache(
    const void* qkv, const void* q, const void* k, const void* v, const float* cos_table,
    const float* sin_table, int32_t max_position, int32_t rotary_dim, int32_t interleaved,
    void* q_out, void* k_cache, void* v_cache, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_new, const int32_t* cu_seqlens_kv,
    int32_t batch, int32_t total_new, int32_t max_seqlen_kv, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size, int32_t num_blocks,
    attn_dtype dtype, void* stream);

/*
 * attn_paged_prefill_fwd -- varlen attention of packed queries against the
 * paged cache: out = softmax(scale * q k^T + mask) v per sequence and head.
 * The fused form of the onnxruntime PR's gather-then-varlen-attention path
 * (section Implementation, steps 2-3), with the masks of the blt issue and
 * the FlexAttention commit.
 *   q            [total_q, num_heads, head_size], dtype ATTN_F16 or ATTN_BF16
 *   k_cache, v_cache, block_table, max_blocks_per_seq, block_size, num_blocks:
 *                the paged cache as above (same dtype as q)
 *   cu_seqlens_q, cu_seqlens_kv  int32 [batch + 1]
 *   max_seqlen_q, max_seqlen_kv  upper bounds of the per-sequence lengths
 *                (host values; they size the launch, no device sync is made)
 *   mask_flags, q_ids, kv_ids    see Conventions (ids may be NULL unless the
 *                matching flag is set)
 *   window_left, softcap         local window and score cap (Conventions)
 *   out          [total_q, num_heads, head_size], same dtype as q
 *   lse          float32 [total_q, num_heads] or NULL
 * Supported: head_size 64 or 128; block_size 16, 32 or 64;
 * num_heads % num_kv_heads == 0.  Errors: NULL pointer, bad shape,
 * unsupported dtype/head_size/block_size/mask, launch failure.
 */
attn_status attn_paged_prefill_fwd(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                   int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                                   int32_t max_seqlen_kv, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t num_blocks,
                                   float scale, uint32_t mask_flags, const int32_t* q_ids,
                                   const int32_t* kv_ids, int32_t window_left, float softcap,
                                   attn_dtype dtype, void* out, float* lse, void* stream);

/*
 * attn_paged_prefill_block_sparse_fwd -- attn_paged_prefill_fwd under a
 * stored block-sparse mask: the BlockMask of FlexAttention as the blt issue's
 * lowering arguments and the FlexAttention commit's test graph show it
 * (partial and full kv-block lists per query block, block sizes, mask_mod),
 * applied per packed varlen sequence.  Query block qb of a sequence is its
 * rows [qb*q_block, (qb+1)*q_block), key block kb its keys
 * [kb*kv_block, (kb+1)*kv_block).  For a (sequence, mask head, query block)
 * the first kv_num_blocks entries of kv_indices are partial blocks, where
 * mask_flags / window_left decide per element, and the first
 * full_kv_num_blocks entries of full_kv_indices are full blocks, visible
 * wherever the key exists (the element mask is not evaluated there, as
 * FlexAttention skips mask_mod on full blocks); every other block is hidden.
 * A block in both lists counts as full.  Ids outside
 * [0, ceil(kv_len / kv_block)) are ignored; counts are clamped to
 * [0, list_capacity].
 *   q_block      power of two, 32 .. 2^30;  kv_block  power of two, 64 .. 2^30
 *   mask_heads   1 (one mask for all heads), num_kv_heads (one per kv head)
 *                or num_heads (one per query head)
 *   num_q_blocks query blocks per sequence in the arrays, at least
 *                ceil(max_seqlen_q / q_block);  list_capacity  entries per list
 *   kv_num_blocks, full_kv_num_blocks  int32 [batch, mask_heads, num_q_blocks]
 *   kv_indices, full_kv_indices  int32 [batch, mask_heads, num_q_blocks,
 *                list_capacity]; the full pair may both be NULL (no full
 *                blocks).  Device memory, read only, owned by the caller.
 * Other arguments as attn_paged_prefill_fwd.  Limit: a workgroup keeps one
 * byte per (query block it touches, key block) in LDS, so
 * max(1, rows / q_block) * ceil(max_seqlen_kv / kv_block) <= 16384 with rows
 * = 256 / (query heads packed per kv head: the largest power of two up to 8
 * dividing num_heads / num_kv_heads, 1 when mask_heads == num_heads);
 * beyond it ATTN_ERR_UNSUPPORTED.  Errors: as attn_paged_prefill_fwd, plus
 * ATTN_ERR_NULL_ARG for a missing list (or half of the full pair),
 * ATTN_ERR_UNSUPPORTED for block sizes, ATTN_ERR_BAD_SHAPE for mask_heads,
 * num_q_blocks or list_capacity.
 */
attn_status attn_paged_prefill_block_sparse_fwd(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
    int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_kv,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, uint32_t mask_flags, const int32_t* q_ids,
    const int32_t* kv_ids, int32_t window_left, float softcap, int32_t q_block, int32_t kv_block,
    int32_t mask_heads, int32_t num_q_blocks, int32_t list_capacity,
    const int32_t* kv_num_blocks, const int32_t* kv_indices, const int32_t* full_kv_num_blocks,
    const int32_t* full_kv_indices, attn_dtype dtype, void* out, float* lse, void* stream);

/*
 * attn_varlen_bwd_workspace_bytes -- workspace attn_varlen_bwd needs: one
 * float per (query row, head), rounded up to 256 bytes.  Host only.
 */
size_t attn_varlen_bwd_workspace_bytes(int32_t total_q, int32_t num_heads);

/*
 * attn_varlen_bwd -- gradients of the varlen attention forward (the backward
 * that the FlexAttention LSE output of the blt issue's kernel options and
 * the varlen function of the vllm-project/flash-attention "Rope dim" review
 * serve).  With P the masked softmax of scale * q k^T, the forward output
 * O = P v, the upstream gradient dO and delta = rowsum(dO * O):
 * dv = P^T dO, dS = P * (dO v^T - delta), dq = scale dS k, dk = scale dS^T q;
 * dk and dv sum over the query heads of each kv head.  P is rebuilt from
 * the forward's lse (natural log, as attn_paged_prefill_fwd returns it).
 * K and V are packed varlen tensors here (training holds them unpaged).
 *   q, out, dout [total_q, num_heads, head_size];  k, v [total_kv,
 *                num_kv_heads, head_size];  lse float32 [total_q, num_heads]
 *   cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, scale,
 *   mask_flags, q_ids, kv_ids, window_left, softcap  as attn_paged_prefill_fwd
 *                (the forward's mask and cap; under a cap c the score is
 *                c tanh(scale q.k / c), so dS also takes its derivative
 *                1 - tanh^2)
 *   dq [total_q, num_heads, head_size], dk, dv [total_kv, num_kv_heads,
 *                head_size]: written whole (rows no key or query reaches get 0)
 *   workspace    device scratch of attn_varlen_bwd_workspace_bytes bytes,
 *                256-byte aligned, owned by the caller, no initialisation;
 *                calls sharing it must not overlap in time
 * dtype ATTN_F16 or ATTN_BF16 for every 16-bit tensor; head_size 64 or 128.
 * All tensors 16-byte aligned device memory.  q, out, dout, lse and dq may
 * be NULL when total_q is 0, k, v, dk and dv when total_kv is 0 (empty
 * tensors); with no query rows and some keys, dk and dv are written as 0.
 * Errors: as attn_paged_prefill_fwd, plus ATTN_ERR_WORKSPACE.
 */
attn_status attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_kv, int32_t batch, int32_t total_q,
                            int32_t total_kv, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            float scale, uint32_t mask_flags, const int32_t* q_ids,
                            const int32_t* kv_ids, int32_t window_left, float softcap,
                            attn_dtype dtype, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * attn_paged_decode_workspace_bytes -- workspace size attn_paged_decode_fwd
 * needs for these sizes (same window_left and split_tokens arguments).  Host
 * only, no HIP call.  Returns 0 for invalid sizes.
 */
size_t attn_paged_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_size, int32_t max_seqlen_kv,
                                         int32_t window_left, int32_t split_tokens);

/*
 * attn_paged_decode_fwd -- one query token per sequence against its paged
 * cache (q_len = 1; under bottom-right alignment the query sees all kv_len
 * keys).  Split-KV: the 32-key tiles of every (sequence, group of up to 4
 * adjacent kv heads) unit are laid end to end and each workgroup takes an
 * equal share of that list, cut into pieces at the units' ends; a second
 * kernel merges each query head's partial results with their logsumexp (the
 * LSE output of the blt issue's kernel options).
 *   q            [batch, num_heads, head_size], ATTN_F16 or ATTN_BF16
 *   cu_seqlens_kv int32 [batch + 1]; max_seqlen_kv bounds every kv length
 *   window_left, softcap  as prefill: the window keeps a sequence's last
 *                window_left keys, and the tiles then cover only those keys
 *   split_tokens keys per workgroup share: a multiple of 256 no larger than
 *                8192, or 0 for equal shares over two workgroups per CU
 *                (at least 512 keys each); the tile list (batch x
 *                kv-head groups x tiles of max_seqlen_kv) must stay within 2^30
 *   out          [batch, num_heads, head_size], same dtype as q
 *   lse          float32 [batch, num_heads] or NULL
 *   workspace    device scratch of at least
 *                attn_paged_decode_workspace_bytes(...) bytes, 256-byte aligned,
 *                owned by the caller; its contents need no initialisation.
 *                Calls that share a workspace must not overlap in time.
 * Errors: as prefill, plus ATTN_ERR_WORKSPACE.
 */
attn_status attn_paged_decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* cu_seqlens_kv, int32_t batch,
                                  int32_t max_seqlen_kv, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_size, int32_t block_size, int32_t num_blocks,
                                  float scale, int32_t window_left, float softcap,
                                  int32_t split_tokens, attn_dtype dtype, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_paged_decode_fwd_noalloc -- attn_paged_decode_fwd for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same computation and
 * arguments without the workspace pair.  The split partials live in a
 * library-owned scratch array of ATTN_DECODE_SCRATCH_BYTES bytes on each GPU
 * (held from the library's first use of that GPU until the process ends).
 * No allocation or free of any kind happens inside the call.
 *   Errors: as attn_paged_decode_fwd; ATTN_ERR_WORKSPACE when these sizes
 *   need more than ATTN_DECODE_SCRATCH_BYTES (the need is
 *   attn_paged_decode_workspace_bytes with the same arguments), checked on
 *   the host before any HIP call.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (two streams, two threads) race and give undefined
 *   results; calls on one stream are ordered and safe.  The scratch keeps
 *   the last call's partials; nothing in it needs to start at zero.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_paged_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, int32_t max_blocks_per_seq,
                                          const int32_t* cu_seqlens_kv, int32_t batch,
                                          int32_t max_seqlen_kv, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_size,
                                          int32_t block_size, int32_t num_blocks, float scale,
                                          int32_t window_left, float softcap,
                                          int32_t split_tokens, attn_dtype dtype, void* out,
                                          float* lse, void* stream);

/*
 * attn_paged_decode_fp8kv_fwd -- attn_paged_decode_fwd over an fp8 e4m3
 * paged cache: the e4m3 format and per-tensor descales of the FlexAttention
 * commit applied to the paged cache of the onnxruntime PR (the combination
 * is this library's, not the pages').  Half the cache bytes per token.
 *   k_cache8, v_cache8  uint8 e4m3 codes [num_blocks, block_size,
 *                num_kv_heads, head_size] (attn_reshape_and_cache with
 *                ATTN_FP8_E4M3 fills them)
 *   kv_descale   float32 [2] (device): real K = kv_descale[0] * decoded code,
 *                real V = kv_descale[1] * decoded code
 *   q_dtype      ATTN_F16 or ATTN_BF16, the dtype of q and out
 *   other arguments, the workspace (attn_paged_decode_workspace_bytes) and the
 *   errors: as attn_paged_decode_fwd.
 * Every e4m3 code is widened exactly to q's 16-bit type; scores, softmax and
 * accumulation in fp32.
 */
attn_status attn_paged_decode_fp8kv_fwd(const void* q, const void* k_cache8, const void* v_cache8,
                                        const float* kv_descale, const int32_t* block_table,
                                        int32_t max_blocks_per_seq, const int32_t* cu_seqlens_kv,
                                        int32_t batch, int32_t max_seqlen_kv, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_size,
                                        int32_t block_size, int32_t num_blocks, float scale,
                                        int32_t window_left, float softcap, int32_t split_tokens,
                                        attn_dtype q_dtype, void* out, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * attn_fp8_fwd -- dense varlen fp8 e4m3 attention with a column-major V.
 * The fp8 path of the FlexAttention commit: Q and K row-major, V column-major
 * so that the fp8 product softmax_scores @ V reads V contiguously along the
 * key dimension (commit message, Context and Fix summary;
 * _enforce_mem_layouts).
 *   q8           uint8 e4m3 codes [total_q, num_heads, head_size]
 *   k8           uint8 e4m3 codes [total_kv, num_kv_heads, head_size]
 *   v8_colmajor  uint8 e4m3 codes [num_kv_heads, head_size, total_kv]
 *   descale_qkv  float32 [3] (device): real value = descale * decoded code
 *   cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, masks,
 *   window_left, softcap: as prefill (the cap applies to the descaled score)
 *   out_bf16     bf16 [total_q, num_heads, head_size]
 *   lse          float32 [total_q, num_heads] or NULL
 * Scores and the softmax run in fp32.  The probabilities are rounded to e4m3
 * (nearest even) for the P.V product, and each row's normaliser is summed
 * from those rounded values.  Supported: head_size 128, total_kv <= 2^27
 * (ATTN_ERR_BAD_SHAPE beyond).  Sequences whose V columns do not start on a
 * 16-key boundary (total_kv or a cu_seqlens_kv entry not a multiple of 16)
 * are supported on a slower load path.
 */
attn_status attn_fp8_fwd(const void* q8, const void* k8, const void* v8_colmajor,
                         const float* descale_qkv, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_kv, int32_t batch, int32_t total_q,
                         int32_t total_kv, int32_t max_seqlen_q, int32_t max_seqlen_kv,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_size, float scale,
                         uint32_t mask_flags, const int32_t* q_ids, const int32_t* kv_ids,
                         int32_t window_left, float softcap, void* out_bf16, float* lse,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CU_SEQLENS_H */
