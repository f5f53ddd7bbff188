/*
 * nv_paged.h - C ABI of the paged-KV hot path for AMD Instinct MI355X (gfx950).
 *
 * The library implements the three device operations a paged-KV inference engine runs in
 * every attention layer, as described in "Nano-vLLM Field Guide", Step 10.3 (attention.py:
 * storing K/V and calling FlashAttention), plus the host-side index metadata of Steps 07.5 to
 * 07.7 (prepare_prefill, prepare_decode, prepare_block_tables):
 *
 *   nv_store_kvcache       scatter this step's new K/V rows into the block-paged pools
 *   nv_paged_attn_prefill  causal varlen prefill attention reading K/V through block tables
 *   nv_paged_attn_decode   one-token decode attention reading K/V through block tables
 *
 * Conventions shared by every call
 *  - "device" pointers must point to memory of the current HIP device; "host" pointers to
 *    ordinary host memory. All device work is enqueued on `stream` and is asynchronous: the
 *    library never synchronises, allocates or frees, and keeps no pointer after returning.
 *    The caller owns every buffer.
 *  - bf16 is the 16-bit brain-float format; values are passed as raw 16-bit patterns.
 *  - K/V pool layout ("Nano-vLLM Field Guide", Step 07.4): one layer's key pool and value pool
 *    are each [num_blocks, block_size, num_kv_heads, head_dim] bf16, contiguous. Flattening the
 *    first two dims gives [num_slots, num_kv_heads * head_dim]: a slot is one row of
 *    D = num_kv_heads * head_dim values, and slot = block_id * block_size + offset (Step 05.1).
 *  - Block tables: int32 [batch, max_blocks_per_seq], row b lists sequence b's physical block
 *    ids in logical order, padded with -1 (Step 07.7). Only the first ceil(L_b / block_size)
 *    entries of a row are read, where L_b is the number of keys the sequence attends to.
 *  - Query head h reads kv head h / (num_heads / num_kv_heads) (the contiguous grouping that
 *    tensor parallelism's head split implies, Step 10.1).
 *  - Errors: arguments that can be checked on the host are checked before anything is
 *    launched; a failed check returns a negative status and enqueues nothing. Contents of
 *    device buffers (slot values, block ids, lengths) are preconditions and are not checked:
 *    a slot outside the pool or a block id outside the pool is undefined behaviour, exactly as
 *    in the engine the pages describe, which asserts shapes only. nv_check_indices() checks
 *    host copies of them.
 */
#ifndef NV_PAGED_H
#define NV_PAGED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NV_OK = 0,
    NV_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes or strides */
    NV_ERR_UNSUPPORTED = -2, /* valid request this library does not implement (e.g. head_dim) */
    NV_ERR_LAUNCH = -3,      /* the HIP runtime rejected a kernel launch */
    NV_ERR_WORKSPACE = -4,   /* decode workspace missing or smaller than required */
    NV_ERR_SCRATCH = -5      /* the library's static scratch is smaller than the call needs */
} nv_status;

/* Static, human-readable name of a status code. Never NULL. */
const char *nv_status_string(nv_status status);

/* ------------------------------------------------------------------------------------------
 * K/V store ("Nano-vLLM Field Guide", Step 10.3, the store kernel and its wrapper).
 *
 * For every token row i in [0, num_tokens) with slot = slot_mapping[i] != -1:
 *   k_cache[slot, :] = key[i, :]  and  v_cache[slot, :] = value[i, :]   (D values, bit copy)
 * Rows whose slot is -1 (padding rows of a captured decode batch) write nothing. It runs
 * before attention in the same step, so attention sees this step's keys.
 *
 *   key, value        device bf16 [num_tokens, num_kv_heads, head_dim]; the last two dims are
 *                     contiguous (head stride head_dim, element stride 1); row i starts at
 *                     element i * key_row_stride (resp. value_row_stride). value may be a view
 *                     into a fused q|k|v projection output, whose rows are wider than D.
 *   k_cache, v_cache  device bf16 pools [num_slots, D], D = num_kv_heads * head_dim.
 *   slot_mapping      device int32 [num_tokens]; -1 or a slot in [0, num_slots).
 * Requirements: row strides >= D; num_tokens >= 0 (0 enqueues nothing). Two rows with the same
 * slot are a precondition violation (each new token owns its slot).
 * ------------------------------------------------------------------------------------------ */
nv_status nv_store_kvcache(const void *key, int64_t key_row_stride,
                           const void *value, int64_t value_row_stride,
                           void *k_cache, void *v_cache,
                           const int32_t *slot_mapping, int64_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                           hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Paged prefill attention ("Nano-vLLM Field Guide", Step 10.3, prefill with cached context,
 * and Step 07.5 for the packed-batch metadata).
 *
 * Sequence b has Lq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] new query rows, packed from row
 * cu_seqlens_q[b] of q, and attends to Lk_b = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys (its
 * cached prefix plus its new tokens, already stored) read through row b of block_tables. Row i
 * of the sequence sees keys 0 .. (Lk_b - Lq_b) + i: the causal mask is aligned to the
 * bottom-right corner, so a prefix-cache hit and a later chunk of a long prompt are the same
 * computation. out[row, h, :] = softmax(softmax_scale * q K^T) V, rounded to bf16 (nearest
 * even).
 *
 *   q              device bf16 [total_q, num_heads, head_dim] contiguous, total_q =
 *                  cu_seqlens_q[batch].
 *   k_cache/v_cache device bf16 pools as above (read only).
 *   cu_seqlens_q/k device int32 [batch + 1], non-decreasing from 0; only differences are used,
 *                  K/V location comes from the block table. Precondition: Lk_b >= Lq_b.
 *   max_seqlen_q   host int >= every Lq_b: sizes the launch without a device round trip.
 *   max_seqlen_k   host int >= every Lk_b.
 *   block_tables   device int32 [batch, max_blocks_per_seq].
 *   softmax_scale  positive and finite; the engine passes head_dim ** -0.5.
 *   out            device bf16 [total_q, num_heads, head_dim] contiguous; may not alias q.
 * Supported: head_dim == 128, num_heads % num_kv_heads == 0, (num_heads / num_kv_heads) <= 8,
 * block_size >= 1, ceil(max_seqlen_k / block_size) <= 2048.
 * block_tables == NULL selects the packed fresh-K/V mode: k_cache/v_cache are then contiguous
 * [total_k, num_kv_heads, head_dim] tensors and the call is nv_attn_prefill_packed with row
 * strides num_kv_heads * head_dim (block_size and max_blocks_per_seq are ignored).
 * ------------------------------------------------------------------------------------------ */
nv_status nv_paged_attn_prefill(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                const int32_t *block_tables, int32_t max_blocks_per_seq,
                                int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, float softmax_scale,
                                void *out, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Prefill attention over packed fresh K/V ("Nano-vLLM Field Guide", Step 10.3: a prefill with
 * no cached context attends over the freshly projected q, k, v, with cu_seqlens describing
 * the packed sequences; Step 07.5 for cu_seqlens).
 *
 * Same operation and mask as nv_paged_attn_prefill, but key j of sequence b is row
 * cu_seqlens_k[b] + j of k and v (no block table). In the engine's fresh prefill
 * cu_seqlens_k == cu_seqlens_q; Lk_b >= Lq_b is the precondition in general.
 *
 *   k, v           device bf16 [total_k, num_kv_heads, head_dim], total_k = cu_seqlens_k[batch];
 *                  the last two dims contiguous (heads head_dim apart).
 *   k_row_stride / v_row_stride  elements between consecutive rows: >= num_kv_heads *
 *                  head_dim and a multiple of 8 (v may be a view into the fused QKV output).
 * Other arguments, layouts, limits and errors as for nv_paged_attn_prefill; additionally
 * NV_ERR_INVALID_ARG for a bad stride.
 * ------------------------------------------------------------------------------------------ */
nv_status nv_attn_prefill_packed(const void *q, const void *k, int64_t k_row_stride,
                                 const void *v, int64_t v_row_stride,
                                 const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                 int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t batch,
                                 int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 float softmax_scale, void *out, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Fused per-head QK RMSNorm + rotary embedding + K/V store ("Nano-vLLM Field Guide", Step 9.5,
 * Qwen3Attention.forward: q_norm / k_norm on every head, rotary_emb on q and k at the token's
 * position, then store_kvcache; the formulas are Step 10.4, layernorm.py, and Step 10.5,
 * rotary_embedding.py).
 *
 * For token t, with its row of the fused projection output qkv[t] = [Hq q heads | Hkv k heads
 * | Hkv v heads] of head_dim values each:
 *   q and k heads x: n = bf16(x * rsqrt(mean(x^2) + eps)), y = bf16(n * w) (w = q_norm_weight
 *   for q heads, k_norm_weight for k heads); then with y1, y2 the two halves of y and the
 *   table row of positions[t]: out = [bf16(y1 cos - y2 sin), bf16(y2 cos + y1 sin)].
 *   q results -> q_out[t]; k results -> k_out[t] (if k_out is not NULL) and to row
 *   slot_mapping[t] of k_cache; v heads unchanged -> row slot_mapping[t] of v_cache.
 *   A slot of -1 stores nothing (q_out and k_out are still written).
 *
 *   qkv            device bf16 [num_tokens, (Hq + 2 Hkv) head_dim] with row stride
 *                  qkv_row_stride (elements, >= that width, multiple of 8).
 *   positions      device int64 [num_tokens]; precondition 0 <= p < max_position (positions
 *                  outside are clamped into the table).
 *   q/k_norm_weight device bf16 [head_dim].
 *   cos_sin_cache  device fp32 [max_position, head_dim]: row p holds cos(p theta_i) for
 *                  i < head_dim/2, then sin(p theta_i) (the engine's table, theta_i =
 *                  base^(-2i/head_dim)); read only.
 *   eps            >= 0 (the engine uses 1e-6).
 *   q_out          device bf16 [num_tokens, Hq, head_dim] contiguous.
 *   k_out          device bf16 [num_tokens, Hkv, head_dim] contiguous, or NULL.
 *   k_cache/v_cache/slot_mapping/num_slots  as for nv_store_kvcache.
 * Alignment: qkv, both norm weights, cos_sin_cache, q_out, k_out (when given), k_cache and
 * v_cache must start on a 16-byte boundary (the kernel moves 16-byte vectors).
 * Supported: head_dim == 128, Hq % Hkv == 0. Errors: NV_ERR_INVALID_ARG (null pointer, bad
 * sizes, stride, eps or a misaligned buffer), NV_ERR_UNSUPPORTED (head_dim), NV_ERR_LAUNCH.
 * ------------------------------------------------------------------------------------------ */
nv_status nv_qk_norm_rope_store(const void *qkv, int64_t qkv_row_stride,
                                const int64_t *positions, const void *q_norm_weight,
                                const void *k_norm_weight, const float *cos_sin_cache,
                                int64_t max_position, float eps, void *q_out, void *k_out,
                                void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                int64_t num_tokens, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int64_t num_slots, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Paged decode attention ("Nano-vLLM Field Guide", Step 10.3, decode; Step 07.6 for
 * context_lens; Step 07.8 for padding rows).
 *
 * One query row per sequence: out[b, h, :] = softmax(softmax_scale * q[b, h] K_b^T) V_b over
 * all context_lens[b] keys of sequence b (they include the token stored in this step). A row
 * with context_lens[b] == 0 (a padding row) attends to nothing and its output is zeros. The
 * key range of each sequence may be split into chunks processed in parallel; the partial
 * results (max, sum, weighted values) are then merged by a log-sum-exp combine. The split
 * length depends only on batch, num_kv_heads, max_blocks_per_seq and block_size; when no row
 * can span two splits a single attention kernel is launched. When the grid is too large to run
 * in one go on the chip, a small kernel first orders the sequences longest first (by bucketed
 * context length) into the workspace, and the attention kernel dispatches them in that order;
 * the order changes no output. The workspace size is 0 only when neither applies.
 *
 *   q             device bf16 [batch, num_heads, head_dim] contiguous.
 *   context_lens  device int32 [batch], 0 <= context_lens[b] <= max_blocks_per_seq*block_size.
 *   block_tables  device int32 [batch, max_blocks_per_seq].
 *   workspace     device scratch of at least nv_paged_attn_decode_workspace_size(...) bytes,
 *                 256-byte aligned, owned by the caller; its contents need no initialisation
 *                 and are garbage afterwards. Calls that run concurrently need separate
 *                 workspaces. May be NULL when the required size is 0.
 *   softmax_scale positive and finite; the engine passes head_dim ** -0.5.
 *   out           device bf16 [batch, num_heads, head_dim] contiguous.
 * Supported: head_dim == 128, num_heads % num_kv_heads == 0, (num_heads / num_kv_heads) <= 8,
 * block_size >= 1. Errors (nothing launched): NV_ERR_INVALID_ARG (null pointer, negative or
 * zero sizes, Hq % Hkv != 0, scale not positive and finite), NV_ERR_UNSUPPORTED (head_dim, a
 * group above 8, batch or num_kv_heads above 65535, more than 65535 splits, or a grid of
 * 2^31 workgroups or more),
 * NV_ERR_WORKSPACE (workspace smaller than required or not 256-byte aligned); NV_ERR_LAUNCH
 * if the launch itself fails. An empty batch returns NV_OK.
 * ------------------------------------------------------------------------------------------ */
size_t nv_paged_attn_decode_workspace_size(int32_t batch, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_blocks_per_seq, int32_t block_size);

nv_status nv_paged_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *context_lens, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, int32_t batch, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               float softmax_scale, void *workspace, size_t workspace_bytes,
                               void *out, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Decode that allocates nothing, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments as nv_paged_attn_decode without the workspace, and the same result bit for
 * bit (the same kernels). The workspace is a static device array of NV_DECODE_SCRATCH_BYTES
 * inside the library: each GPU the library runs on holds its own copy from the first call on
 * that GPU until the process ends. The call allocates and frees nothing. Every call on one GPU
 * shares that GPU's array and leaves garbage in it (no call needs it zeroed), so calls that
 * overlap on one GPU (different streams or threads at the same time) race: issue them one
 * after another, e.g. on one stream. The device is the current one; `stream` must belong to it.
 * Errors: as nv_paged_attn_decode, and NV_ERR_SCRATCH, with nothing launched, when the call
 * needs more than NV_DECODE_SCRATCH_BYTES of workspace (nv_paged_attn_decode_workspace_size()
 * tells beforehand; e.g. batch 256 x 16 q heads over 4096-key contexts needs about 4 MiB).
 * NV_ERR_LAUNCH also covers a failed lookup of the array's device address.
 * ------------------------------------------------------------------------------------------ */
#define NV_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

nv_status nv_paged_attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *context_lens, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, int32_t batch,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, float softmax_scale, void *out,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Store + decode in one launch ("Nano-vLLM Field Guide", Step 10.3: store_kvcache, then
 * flash_attn_with_kvcache, for a step of decode rows only).
 *
 * Same result as nv_store_kvcache(key, key_row_stride, value, value_row_stride, k_cache,
 * v_cache, slot_mapping, batch, num_kv_heads, head_dim, num_slots) followed by
 * nv_paged_attn_decode(q, k_cache, v_cache, context_lens, ..., out), bit for bit, provided
 * that (as for every decode step of the engine) slot_mapping[b] is the pool row of key
 * context_lens[b] - 1 of row b, and -1 for rows with context_lens[b] == 0, and that no other
 * row's table reaches that pool row (a shared prefix block is always full, so the block that
 * takes a new token belongs to one sequence). Row b's new key and value (row b of key / value)
 * are written to the pools and used directly as key context_lens[b] - 1 of the attention, so
 * no store kernel runs before it.
 *
 *   key, value          device bf16 [batch, num_kv_heads, head_dim] rows with the given row
 *                       strides (elements), as for nv_store_kvcache; value may be a view into
 *                       the fused QKV output.
 *   slot_mapping        device int32 [batch]; -1 stores nothing.
 *   k_cache, v_cache    the pools, written at the slots and read by the attention.
 *   num_slots           rows of each pool (host-side argument check only).
 *   counters            optional device uint32 [num_counters], num_counters >= batch *
 *                       num_kv_heads, entry b * num_kv_heads + g for row b, kv head g. Given,
 *                       the split kernel also merges the splits of a split row (the last of
 *                       its workgroups to finish merges), so no merge kernel runs and the call
 *                       is one launch. The entries must be zero before the call, and the call
 *                       leaves them zero; the layout does not depend on anything but batch
 *                       and num_kv_heads, so one zeroed array serves calls of any batch up to
 *                       its size (and is untouched by calls that do not split). Calls that run
 *                       concurrently need separate arrays. NULL: the merge kernel runs.
 *   others              as for nv_paged_attn_decode (the same workspace size applies).
 * The output is the same bit for bit with or without counters. With rows that are not 16-byte
 * aligned, or max_blocks_per_seq == 0, the call runs the two calls above one after the other
 * (counters untouched). Errors: as the two calls, and NV_ERR_INVALID_ARG for counters that
 * are too short or not 4-byte aligned.
 * ------------------------------------------------------------------------------------------ */
nv_status nv_paged_attn_decode_store(const void *q, const void *key, int64_t key_row_stride,
                                     const void *value, int64_t value_row_stride,
                                     const int32_t *slot_mapping, void *k_cache, void *v_cache,
                                     int64_t num_slots, const int32_t *context_lens,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, float softmax_scale,
                                     void *workspace, size_t workspace_bytes,
                                     uint32_t *counters, int64_t num_counters, void *out,
                                     hipStream_t stream);

/* Number of keys one decode work item covers for this launch shape (a multiple of 64): the
 * split the decode call uses. Exposed for tests and measurement. */
int32_t nv_paged_attn_decode_split_keys(int32_t batch, int32_t num_kv_heads,
                                        int32_t max_blocks_per_seq, int32_t block_size);

/* ------------------------------------------------------------------------------------------
 * Host-side index metadata ("Nano-vLLM Field Guide", Step 07.5 prepare_prefill, Step 07.6
 * prepare_decode, Step 07.7 prepare_block_tables). All pointers are HOST pointers.
 *
 * A batch of sequences is described by, per sequence b: num_cached[b] tokens already in the
 * cache, num_new[b] tokens computed this step (positions [num_cached, num_cached + num_new)),
 * and its block table: block_ids[table_offsets[b] .. table_offsets[b+1]) (table_offsets has
 * batch + 1 entries, starting at 0).
 * ------------------------------------------------------------------------------------------ */

/* Prefill metadata. Outputs:
 *   slot_mapping  [sum num_new]: slot of every new token, sequence by sequence, position order.
 *   cu_seqlens_q  [batch + 1]: running sum of num_new.
 *   cu_seqlens_k  [batch + 1]: running sum of num_cached + num_new.
 *   max_seqlen_q, max_seqlen_k: largest num_new, largest num_cached + num_new.
 *   block_tables  [batch, bt_width]: tables padded with -1; bt_width >= every table length.
 *   has_cached_context: 1 if cu_seqlens_k[batch] > cu_seqlens_q[batch] (some sequence has cached
 *                 context), else 0; any output pointer except slot_mapping/cu_* may be NULL.
 * Returns NV_ERR_INVALID_ARG if a table is too short for its positions or too wide. */
nv_status nv_prepare_prefill(const int32_t *num_cached, const int32_t *num_new,
                             const int32_t *table_offsets, const int32_t *block_ids,
                             int32_t batch, int32_t block_size,
                             int32_t *slot_mapping, int32_t *cu_seqlens_q, int32_t *cu_seqlens_k,
                             int32_t *max_seqlen_q, int32_t *max_seqlen_k,
                             int32_t *block_tables, int32_t bt_width,
                             int32_t *has_cached_context);

/* Decode metadata, one row per sequence; num_new[b] must be 1, or 0 together with
 * num_cached[b] == 0 for a padding row. Outputs:
 *   slot_mapping [batch]: slot of position len - 1 (len = num_cached + 1); -1 for padding.
 *   context_lens [batch]: len (it includes the token stored this step); 0 for padding.
 *   block_tables [batch, bt_width]: padded with -1. */
nv_status nv_prepare_decode(const int32_t *num_cached, const int32_t *num_new,
                            const int32_t *table_offsets, const int32_t *block_ids,
                            int32_t batch, int32_t block_size,
                            int32_t *slot_mapping, int32_t *context_lens,
                            int32_t *block_tables, int32_t bt_width);

/* Host check of index preconditions on host copies (debug aid; not on the hot path).
 * Checks that every slot is -1 or in [0, num_slots) and that no slot repeats; that every
 * table entry a sequence reads (the first ceil(len / block_size)) is in [0, num_blocks).
 * lens[b] is the number of keys sequence b reads. Returns NV_OK or NV_ERR_INVALID_ARG and, if
 * bad_index is not NULL, the first offending index (slot row, or b * max_blocks_per_seq + j). */
nv_status nv_check_indices(const int32_t *slot_mapping, int64_t num_tokens, int64_t num_slots,
                           const int32_t *block_tables, const int32_t *lens, int32_t batch,
                           int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                           int64_t *bad_index);

#ifdef __cplusplus
}
#endif

#endif /* NV_PAGED_H */
