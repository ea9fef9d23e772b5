/*
 * pa.h - paged grouped-query attention over a block-table fp16 KV cache, for AMD MI355X (gfx950).
 *
 * A C ABI over device pointers. These operations make up the path:
 *   pa_kv_append        fused rotary + scatter of new K/V rows into cache slots
 *   pa_paged_attention  paged attention (decode and chunked prefill), split-KV when useful
 *   pa_paged_attention_noalloc  the same with the library's static scratch (no workspace)
 *   pa_split_combine    log-sum-exp merge of (o, m, l) partials
 *   pa_sparse_forward   fp32 block-sparse "edge" forward emitting (o, m, l) partials
 *   pa_kv_append_rotate_query  the append plus the same rotation of the new query rows
 *   pa_sparse_forward_causal   the sparse forward with a per-row causal key limit
 *   pa_sparse_build_edges      the sparse forward's edge list from a kept-block mask
 *   pa_kv_append_bnsh          the append into a contiguous BNSH cache (the append page's own)
 *   pa_append_attention        the append and the attention in one call (the manifest's op)
 *   pa_check_paged_indices     a debug check of the paged calls' device-resident indices
 *
 * Sources. Argument names and layouts follow three web pages:
 *   [manifest] "com.microsoft.PagedAttention ... manifest.json": the op's inputs, outputs,
 *              attributes, derived shapes, tunables and its scatter / split-attend / merge passes.
 *   [append]   "com.microsoft.SparseAttention ... sparse-kv-append.wgsl.jinja": the KV append
 *              pass with rotary (rotary macros and main).
 *   [sparse]   "alice-llm ... sparse_attention_forward.wgsl": the KV-outer block-sparse forward,
 *              its Params struct, bindings and partial layout.
 *
 * Conventions that hold for every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library never allocates
 *     or frees device memory; scratch space comes in as `workspace`. The one exception is
 *     pa_paged_attention_noalloc, whose scratch is a static array that the library's code object
 *     holds on each device it runs on until the process ends.
 *   - Calls are asynchronous: they validate, enqueue kernels on `stream` (a hipStream_t; NULL is
 *     the null stream) and return. Results are ready when the stream reaches them.
 *   - Host-visible scalars and null pointers are checked before anything is enqueued; a failed
 *     check returns a non-zero pa_status and enqueues nothing. The contents of device-resident
 *     index arrays (cumulative_sequence_length, past_seqlens, block_table, slot_mapping,
 *     edge_meta, block_tables) are the caller's contract and are not checked; the paged ones
 *     can be checked on the device beforehand with pa_check_paged_indices.
 *   - fp16 is IEEE binary16 (`_Float16` / `__half`); element offsets may exceed 2^31.
 *   - The library holds no mutable host state except per-device caches (the compute-unit count,
 *     the address of pa_paged_attention_noalloc's scratch) and the optional timing records
 *     (pa_timing_*). Calls may come from several host threads.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
#define PA_OK 0
#define PA_ERR_NULL 1        /* a required pointer is NULL                                   */
#define PA_ERR_SHAPE 2       /* sizes or attributes violate the op's contract                */
#define PA_ERR_UNSUPPORTED 3 /* a legal configuration this build does not implement          */
#define PA_ERR_WORKSPACE 4   /* workspace smaller than the matching *_workspace_size query   */
#define PA_ERR_HIP 5         /* the HIP runtime reported an error while enqueueing           */

#define PA_ROTARY_NONE 0
#define PA_ROTARY_NEOX 1         /* component d pairs with d + R/2 ([append] rotary macros)  */
#define PA_ROTARY_INTERLEAVED 2  /* component 2i pairs with 2i + 1                            */

#define PA_F16 0
#define PA_F32 1

#define PA_SPLITS_AUTO 0         /* chunk keys chosen on the device from lengths and CU count */
#define PA_SPLITS_PAGE_RULE (-1) /* the manifest's numSplits rule, see pa_paged_attention     */

/*
 * Host-side shape of one paged call. The fields are the manifest's "derive" quantities:
 * tokenCount = dim0(query), blockSize = dim1(key_cache), headSize = dim3(key_cache),
 * maxBlocks = dim1(block_table), batchSize = dim0(cumulative_sequence_length) - 1, and the
 * required attributes num_heads and kv_num_heads.
 */
typedef struct pa_paged_shape {
    int32_t batch;        /* B  >= 1                                                          */
    int32_t num_tokens;   /* T  >= 0: rows of query (all sequences' new tokens, concatenated) */
    int32_t num_heads;    /* H  > 0                                                           */
    int32_t kv_num_heads; /* G  > 0, H % G == 0; query head h reads kv head h / (H / G)        */
    int32_t head_size;    /* D  in {64, 128, 256}                                             */
    int32_t num_blocks;   /* NB >= 1: dim0 of key_cache and value_cache                       */
    int32_t block_size;   /* bs >= 1: tokens per cache block                                  */
    int32_t max_blocks;   /* MB >= 1: block_table row length                                  */
    int32_t packed_qkv;   /* 1: query rows are [Q | K | V] of width (H + 2G) * D and key/value
                             are NULL ([manifest] packedKv); 0: query rows are H * D wide      */
} pa_paged_shape;

/*
 * pa_kv_append - write the new K/V rows of every sequence into their cache slots.
 *
 * Defined by [manifest] pass "scatter" (PagedAttention.ScatterKV: derived-slot and slot_mapping
 * variants) fused with [append] "main": the key is rotated at its own absolute position before
 * it enters the cache, so the cache holds post-rotary keys; values are copied.
 *
 * Row i = cu[b] + t (t < n_b = cu[b+1] - cu[b]) of sequence b sits at position
 * pos = past_seqlens[b] + t. Its slot is slot_mapping[i] when slot_mapping is non-NULL, else
 * block_table[b][pos / bs] * bs + pos % bs. A negative slot writes nothing. For every kv head g
 * the row lands at key_cache[slot / bs][slot % bs][g][:] (same for value_cache). No other cache
 * element is written.
 *
 *   query       fp16 [T, (H+2G)*D] when packed (K at column H*D + g*D, V at (H+G)*D + g*D);
 *               ignored (may be NULL) when not packed
 *   key, value  fp16 [T, G*D]; both NULL when packed, both non-NULL otherwise
 *   key_cache, value_cache  fp16 [NB, bs, G, D], updated in place
 *   cumulative_sequence_length  int32 [B+1], non-decreasing, cu[0] = 0, cu[B] = T
 *   past_seqlens  int32 [B] >= 0
 *   block_table   int32 [B, MB]; entries a sequence uses must lie in [0, NB)
 *   slot_mapping  int32 [T] or NULL; slots must lie in [-inf, NB*bs) and be distinct
 *   cos_cache, sin_cache  fp16 [rotary_positions, rotary_dim/2], row = position; NULL when
 *               rotary_mode == PA_ROTARY_NONE. Every pos must be < rotary_positions.
 *   rotary_dim  even, 0 < rotary_dim <= D when rotary is on (components d >= rotary_dim are
 *               copied); ignored when off
 *   rotary_mode PA_ROTARY_NONE / PA_ROTARY_NEOX / PA_ROTARY_INTERLEAVED
 *
 * Rotary arithmetic: two float32 products (each rounded), one float32 add or subtract, then
 * round-to-nearest-even to fp16; the first member of a pair subtracts its partner's sine term.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (D not 64/128/256, G*D >= 2^24,
 * bs*G*D >= 2^32: the shape limits every paged entry shares), PA_ERR_HIP.
 */
pa_status pa_kv_append(const pa_paged_shape *shape, const void *query, const void *key,
                       const void *value, void *key_cache, void *value_cache,
                       const int32_t *cumulative_sequence_length, const int32_t *past_seqlens,
                       const int32_t *block_table, const int32_t *slot_mapping,
                       const void *cos_cache, const void *sin_cache, int32_t rotary_dim,
                       int32_t rotary_mode, int32_t rotary_positions, void *stream);

/*
 * pa_kv_append_rotate_query - pa_kv_append, plus every new query row rotated at its position.
 *
 * The pages rotate only keys in the append and hand queries to attention already positioned
 * ([append] rotary macros and main; [manifest] attention binds no cos/sin). This entry applies
 * the same per-pair rotation, with the same cos/sin rows, to each of the H query head rows of
 * new token t of sequence b at pos = past_seqlens[b] + t, in the same launch as the key/value
 * append. Components d >= rotary_dim are copied; with PA_ROTARY_NONE the rows are copied.
 *   query   required: packed rows (packed_qkv = 1; the Q part is rotated) or fp16 [T, H*D]
 *   q_out   fp16 [T, H*D], caller-owned, every row written; must not be the query buffer
 *           (attention then reads q_out with packed_qkv = 0)
 *   other arguments as pa_kv_append
 * Errors: as pa_kv_append; PA_ERR_NULL when query or q_out is NULL; PA_ERR_SHAPE when
 * q_out == query.
 */
pa_status pa_kv_append_rotate_query(const pa_paged_shape *shape, const void *query,
                                    const void *key, const void *value, void *key_cache,
                                    void *value_cache, const int32_t *cumulative_sequence_length,
                                    const int32_t *past_seqlens, const int32_t *block_table,
                                    const int32_t *slot_mapping, const void *cos_cache,
                                    const void *sin_cache, int32_t rotary_dim,
                                    int32_t rotary_mode, int32_t rotary_positions, void *q_out,
                                    void *stream);

/*
 * Bytes of device workspace pa_paged_attention needs for this shape and split policy (an upper
 * bound that does not depend on device data). Returns 0 for an invalid shape.
 */
size_t pa_paged_attention_workspace_size(const pa_paged_shape *shape, int32_t num_splits);

/*
 * pa_paged_attention - causal paged GQA attention of every query row over its sequence's cache.
 *
 * Defined by [manifest] passes "main" (PagedAttention.Attend), "split_attention"
 * (PagedAttention.AttendSplitK) and "merge" (PagedAttention.AttendSplitKMerge). Reads only the
 * caches: enqueue pa_kv_append first on the same stream so the new rows are present.
 *
 * Query head h of row i (sequence b, position pos = past_b + i - cu[b]) attends with kv head
 * g = h / (H/G) to keys j < limit, limit = pos + 1 when causal, else past_b + n_b. Key j of
 * sequence b is key_cache[block_table[b][j / bs]][j % bs][g][:]. With s_j = (q . k_j) * scale:
 *   output[i][h*D + d] = sum_j exp(s_j - max s) v_j[d] / sum_j exp(s_j - max s), as fp16.
 *
 *   query    fp16, row stride H*D, or (H+2G)*D when shape->packed_qkv (Q in the first H*D)
 *   scale    > 0, or <= 0 for 1/sqrt(D)
 *   causal   1 (the manifest's only value) or 0 (every row sees its sequence's whole cache)
 *   num_splits  PA_SPLITS_AUTO: the key range of decode-like rows is cut into chunks whose size
 *            the device picks from the sequence lengths and the CU count;
 *            PA_SPLITS_PAGE_RULE: S = max(1, min(cap, ceil(1024 / (T*G)))) with
 *            cap = max(1, min(16, MB*bs / 128)) ([manifest] numSplits with MAX_SPLITS 16,
 *            SPLIT_MIN_KEYS 128, SPLIT_TARGET_WORKGROUPS 1024);
 *            S >= 1: every decode-like row's keys are cut into at most S chunks.
 *            Split partials are merged in float32 by log-sum-exp; the result does not depend on
 *            the split beyond float32 rounding.
 *   workspace, workspace_bytes  device scratch of at least
 *            pa_paged_attention_workspace_size(shape, num_splits) bytes, 256-byte aligned
 *   output   fp16 [T, H*D]
 * Rows of a sequence with n_b * Qg <= 16 (<= 32 or 64 for Qg above 16 or 32) are decode-like
 * and split-KV eligible; longer sequences run on the chunked-prefill path as items of 128
 * (token, head) columns (128 / Qg tokens of one head group), each covering its causal key range
 * in one pass. Qg = H/G, except that a kv head with more than 64 query heads (more than 16 at
 * D = 256) is served as several groups of at most Qg = 16 heads that read the same cache head.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (the shape limits of pa_kv_append),
 * PA_ERR_WORKSPACE, PA_ERR_HIP.
 */
pa_status pa_paged_attention(const pa_paged_shape *shape, const void *query,
                             const void *key_cache, const void *value_cache,
                             const int32_t *cumulative_sequence_length,
                             const int32_t *past_seqlens, const int32_t *block_table, float scale,
                             int32_t causal, int32_t num_splits, void *workspace,
                             size_t workspace_bytes, void *output, void *stream);

/*
 * pa_paged_attention_noalloc - pa_paged_attention without a caller workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.
 *
 * Same arguments, kernels and results (bit for bit) as pa_paged_attention with that call's
 * workspace replaced by a static device array of PA_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each device. The first call on a device looks the array's address up (with that
 * device current); no call allocates, frees or clears memory. Every kernel input in the array
 * is written by the call itself (the planner zeroes its counters), so the previous call's
 * contents never matter.
 * Calls that overlap on one device (two streams, or two host threads, with no ordering between
 * them) share the array and race: order them on one stream, or use pa_paged_attention with
 * separate workspaces.
 * Errors: those of pa_paged_attention; PA_ERR_WORKSPACE when
 * pa_paged_attention_workspace_size(shape, num_splits) exceeds PA_NOALLOC_SCRATCH_BYTES
 * (checked before any HIP call); PA_ERR_HIP when the address lookup fails.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status pa_paged_attention_noalloc(const pa_paged_shape *shape, const void *query,
                                     const void *key_cache, const void *value_cache,
                                     const int32_t *cumulative_sequence_length,
                                     const int32_t *past_seqlens, const int32_t *block_table,
                                     float scale, int32_t causal, int32_t num_splits,
                                     void *output, void *stream);

/*
 * pa_append_attention - the whole op of [manifest]: pass "scatter" and then the attention
 * passes ("main", "split_attention", "merge"), in one call.
 *
 * Same results, bit for bit, as pa_kv_append (q_out NULL) or pa_kv_append_rotate_query (q_out
 * given) followed on the same stream by pa_paged_attention over the query as passed (q_out
 * NULL) or over q_out as fp16 [T, H*D] rows (q_out given). The append and the attention's
 * planner share one launch: the planner reads only cumulative_sequence_length and past_seqlens,
 * which the append does not write.
 *   query     required; packed rows (shape->packed_qkv = 1) or fp16 [T, H*D]
 *   key, value, key_cache, value_cache, cumulative_sequence_length, past_seqlens,
 *   block_table, slot_mapping, cos_cache, sin_cache, rotary_dim, rotary_mode,
 *   rotary_positions  as pa_kv_append (block_table is required here: attention reads it)
 *   q_out     NULL, or fp16 [T, H*D] for the rotated query rows as pa_kv_append_rotate_query
 *   scale, causal, num_splits, workspace, workspace_bytes, output  as pa_paged_attention
 *             (the workspace size is pa_paged_attention_workspace_size(shape, num_splits))
 * Every argument of both parts is checked before anything is enqueued.
 * Errors: the union of those of pa_kv_append_rotate_query and pa_paged_attention;
 * PA_ERR_NULL when query is NULL; PA_ERR_SHAPE when q_out == query.
 */
pa_status pa_append_attention(const pa_paged_shape *shape, const void *query, const void *key,
                              const void *value, void *key_cache, void *value_cache,
                              const int32_t *cumulative_sequence_length,
                              const int32_t *past_seqlens, const int32_t *block_table,
                              const int32_t *slot_mapping, const void *cos_cache,
                              const void *sin_cache, int32_t rotary_dim, int32_t rotary_mode,
                              int32_t rotary_positions, void *q_out, float scale,
                              int32_t causal, int32_t num_splits, void *workspace,
                              size_t workspace_bytes, void *output, void *stream);

/*
 * pa_split_combine - log-sum-exp merge of partial attention results.
 *
 * The merge of [manifest] pass "merge" (PagedAttention.AttendSplitKMerge, partialOut /
 * partialStats intermediates) and of the per-edge partials of [sparse] (ForwardPartials).
 * Group k owns partial units e in [group_ptr[k], group_ptr[k+1]) when group_ptr is non-NULL,
 * else [k*num_splits, (k+1)*num_splits). Unit e holds `lanes` partials p = e*lanes + lane:
 * o_partial[p*head_dim + d], m_partial[p] (a natural-log max), l_partial[p] (a sum of exp).
 * Output row r = k*lanes + lane:
 *   M = max m_p over units with l_p > 0; w = exp(m_p - M) (0 when l_p <= 0);
 *   out[r][d] = sum w o_p[d] / sum w l_p, or 0 when no unit has l_p > 0.
 *   out_dtype PA_F16 (round to nearest even) or PA_F32; out is [num_groups*lanes, head_dim].
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_groups < 0, lanes < 1, head_dim not a positive
 * multiple of 4, num_splits < 1 without group_ptr), PA_ERR_UNSUPPORTED (head_dim not 64, 128
 * or 256), PA_ERR_HIP.
 */
pa_status pa_split_combine(const float *o_partial, const float *m_partial,
                           const float *l_partial, const int32_t *group_ptr, int32_t num_groups,
                           int32_t lanes, int32_t num_splits, int32_t head_dim, int32_t out_dtype,
                           void *out, void *stream);

/*
 * Shape of one block-sparse call: [sparse] Params (total_partials = num_edges * qhead, qhead,
 * head_dim, block_size, page_size, pages_per_block = block_size / page_size, hkv,
 * hq = hkv * qhead, max_pages) plus the sizes of the bound arrays.
 */
typedef struct pa_sparse_shape {
    int32_t num_edges;  /* E >= 0                                                     */
    int32_t tq;         /* rows of q_buf                                              */
    int32_t hkv;        /* kv heads                                                   */
    int32_t qhead;      /* query heads per kv head (the q-head lanes of an edge)      */
    int32_t head_dim;   /* D in {64, 128, 256}                                        */
    int32_t block_size; /* keys per sparse block, multiple of page_size, <= 128 (<= 64
                           at D = 256)                                                */
    int32_t page_size;  /* keys per page                                              */
    int32_t num_pages;  /* dim0 of k_pages / v_pages                                  */
    int32_t max_pages;  /* block_tables row length                                    */
    int32_t batch;      /* block_tables rows                                          */
} pa_sparse_shape;

/* Bytes of device workspace pa_sparse_forward needs (0 for an invalid shape). */
size_t pa_sparse_forward_workspace_size(const pa_sparse_shape *shape);

/*
 * pa_sparse_forward - one (o, m, l) partial per (edge, q-head lane), in fp32.
 *
 * Defined by [sparse] sparse_forward. Edge e is edge_meta[5e..5e+4] = (q_idx, h, blk, batch,
 * block_len), with 0 <= block_len <= block_size (the page's host clamps it to the block). Lane
 * qh of edge e reads query row q_buf[q_idx][h*qhead + qh][:] and keys t < block_len of block
 * blk: page id block_tables[batch][blk*(block_size/page_size) + t/page_size], row
 * k_pages[page][h][t % page_size][:]. An unmapped page (id < 0) contributes no key. With
 * s_t = (q . k_t) * softmax_scale over the mapped keys:
 *   m = max s_t, l = sum exp(s_t - m), o[d] = sum exp(s_t - m) v_t[d]   (not normalised)
 * written at p = e*qhead + qh: o_partial[p*D + d], m_partial[p], l_partial[p]. An edge with
 * block_len <= 0 or no mapped key writes the sentinel o = 0, m = -1e30, l = 0.
 *   q_buf   f32 [tq, hkv*qhead, D];  k_pages, v_pages  f32 [num_pages, hkv, page_size, D]
 *   edge_meta int32 [E, 5];  block_tables int32 [batch, max_pages]
 *   causal  must be 0: the page leaves the right-aligned causal mask unimplemented (the mask
 *           needs each row's key position: pa_sparse_forward_causal)
 *   workspace  at least pa_sparse_forward_workspace_size(shape) bytes, 256-byte aligned
 * Edges may come in any order; the kernel groups them by (batch, h, blk) so each block of keys
 * is read once per group. Merge the partials with pa_split_combine.
 * Accuracy: the products run on fp16 matrix instructions over hi + lo splits of operands
 * scaled by powers of two (each query row, each key block, each value dimension outside
 * [0.5, 2^15)), 22 significant bits per element, or an absolute error bound for elements far
 * below their group's maximum; the partials are tested against an fp64 evaluation at 1e-4
 * (relative to max(1, |value|)), including outlier channels and magnitudes down to 1e-39.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (causal != 0, D not 64/128/256,
 * block_size > 128, or > 64 at D = 256), PA_ERR_WORKSPACE, PA_ERR_HIP.
 */
pa_status pa_sparse_forward(const pa_sparse_shape *shape, const float *q_buf,
                            const float *k_pages, const float *v_pages,
                            const int32_t *edge_meta, const int32_t *block_tables,
                            float softmax_scale, int32_t causal, void *workspace,
                            size_t workspace_bytes, float *o_partial, float *m_partial,
                            float *l_partial, void *stream);

/*
 * pa_sparse_forward_causal - pa_sparse_forward with the right-aligned causal mask that the
 * [sparse] page lists as unimplemented (its header: the host must set causal = 0).
 *
 * q_pos  int32 [tq]: the absolute key position of each query row; key t of an edge's block is
 *        seen only when blk*block_size + t <= q_pos[q_idx], otherwise it is excluded like a key
 *        on an unmapped page. Right-aligned rows of a batch with Tq_b rows and used_b keys have
 *        q_pos = used_b - Tq_b + j for row j. An edge with no key left writes the sentinel.
 * Other arguments, layouts and the workspace size are those of pa_sparse_forward.
 * Errors: as pa_sparse_forward; PA_ERR_NULL when q_pos is NULL and num_edges > 0.
 */
pa_status pa_sparse_forward_causal(const pa_sparse_shape *shape, const float *q_buf,
                                   const float *k_pages, const float *v_pages,
                                   const int32_t *edge_meta, const int32_t *block_tables,
                                   const int32_t *q_pos, float softmax_scale, void *workspace,
                                   size_t workspace_bytes, float *o_partial, float *m_partial,
                                   float *l_partial, void *stream);

/*
 * pa_sparse_build_edges - the edge list of pa_sparse_forward, built on the device from a mask.
 *
 * The [sparse] page's host prepares edge_meta on the CPU (its layout notes: block_len computed
 * from used_kv_lens, clamped by the block). Rows (q, h) are taken in order and blocks in order
 * within a row; every nonzero block_mask[q][h][blk] gives the edge
 *   (q, h, blk, b = q_batch[q], block_len = clamp(used_kv_lens[b] - blk*block_size, 0, block_size))
 * and group_ptr[q*hkv + h] is the index of row (q, h)'s first edge; group_ptr[tq*hkv] is the edge
 * count E. The list is sorted by (q_idx, h, blk) and group_ptr is the CSR offset array that
 * pa_split_combine takes to merge each row's partials.
 *   block_mask    uint8 [tq, hkv, nblk], nonzero = keep
 *   q_batch       int32 [tq], the batch of each query row (an entry outside [0, batch) is
 *                 written as given and reads used_kv_lens of a clamped index)
 *   used_kv_lens  int32 [batch]
 *   edge_meta     int32 [edge_capacity, 5]: edges with index >= edge_capacity are not written
 *                 (E is still counted: read group_ptr[tq*hkv] to size the forward)
 *   group_ptr     int32 [tq*hkv + 1]
 *   workspace     pa_sparse_build_edges_workspace_size(tq, hkv) bytes, 256-byte aligned
 * The edge count lives in device memory: the caller reads it back before sizing
 * pa_sparse_forward's num_edges.
 * Errors: PA_ERR_SHAPE (negative sizes), PA_ERR_UNSUPPORTED (tq*hkv*nblk >= 2^31),
 * PA_ERR_NULL, PA_ERR_WORKSPACE, PA_ERR_HIP.
 */
size_t pa_sparse_build_edges_workspace_size(int32_t tq, int32_t hkv);
pa_status pa_sparse_build_edges(int32_t tq, int32_t hkv, int32_t nblk, int32_t block_size,
                                int32_t batch, const uint8_t *block_mask,
                                const int32_t *q_batch, const int32_t *used_kv_lens,
                                int64_t edge_capacity, int32_t *edge_meta, int32_t *group_ptr,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Shape of a contiguous-cache append: the [append] page's own layout, one padded batch of
 * seq_len new tokens per sequence and a BNSH cache [batch, kv_num_heads, max_cache_seq,
 * head_size] (present_key / present_value, the same allocation as past_key / past_value).
 */
typedef struct pa_bnsh_shape {
    int32_t batch;          /* B >= 1                                                    */
    int32_t seq_len;        /* S: new tokens per sequence (padded), >= 0                 */
    int32_t num_heads;      /* H (packed rows carry H query heads first)                 */
    int32_t kv_num_heads;   /* KVH, H % KVH == 0                                         */
    int32_t head_size;      /* D in {64, 128, 256}                                       */
    int32_t max_cache_seq;  /* positions per (batch, kv head) in the cache               */
    int32_t packed_qkv;     /* 1: query rows are [Q|K|V], key/value == NULL              */
} pa_bnsh_shape;

/*
 * pa_kv_append_bnsh - the [append] page's KV append pass over a contiguous BNSH cache.
 *
 * One write per (batch b, kv head h, new token t < S, component d) at
 * present[((b*KVH + h)*max_cache_seq + past_b + t)*D + d], with the page's padded-batch rule
 * (past-length macro): past_b = 0 when total_sequence_length[0] == S (a prompt), else
 * key_total_sequence_lengths[b] - S, or 0 when that total is below S. The key is rotated at its
 * position exactly as in pa_kv_append; the value is copied. Source row of (b, t):
 * b*S + t of query (packed) or key / value [B*S, KVH*D].
 *   total_sequence_length       int32 [1] (device)
 *   key_total_sequence_lengths  int32 [B] (device)
 *   cos_cache, sin_cache, rotary_dim, rotary_mode, rotary_positions: as pa_kv_append
 * A row whose position is >= max_cache_seq (or >= rotary_positions with rotary on) is not
 * written (the page leaves the bound to its caller).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (D not 64/128/256), PA_ERR_HIP.
 */
pa_status pa_kv_append_bnsh(const pa_bnsh_shape *shape, const void *query, const void *key,
                            const void *value, void *present_key, void *present_value,
                            const int32_t *total_sequence_length,
                            const int32_t *key_total_sequence_lengths, const void *cos_cache,
                            const void *sin_cache, int32_t rotary_dim, int32_t rotary_mode,
                            int32_t rotary_positions, void *stream);

/*
 * pa_check_paged_indices - check the device-resident index contents of a paged call (a debug
 * aid; the other entry points do not check them).
 *
 * The arrays are the [manifest] inputs cumulative_sequence_length, past_seqlens, block_table
 * and slot_mapping, with the sizes its "derive" section fixes from `shape`. The append and the
 * attention kernels follow these indices without bounds checks; this call verifies every rule
 * they rely on and ORs one PA_CHECK_* bit per violated rule into flags[0]:
 *   PA_CHECK_CU_START     cumulative_sequence_length[0] != 0
 *   PA_CHECK_CU_ORDER     cumulative_sequence_length decreases somewhere
 *   PA_CHECK_CU_END       cumulative_sequence_length[B] != num_tokens
 *   PA_CHECK_PAST         a past_seqlens entry is negative
 *   PA_CHECK_TABLE_WIDTH  a sequence's keys (past + new) need more than max_blocks blocks
 *   PA_CHECK_TABLE_ENTRY  a block_table entry that covers one of its sequence's keys lies
 *                         outside [0, num_blocks) (entries past the keys are never read)
 *   PA_CHECK_SLOT         a slot_mapping entry is >= num_blocks * block_size (negative
 *                         entries mean "not written" and pass)
 *   PA_CHECK_SLOT_TABLE   a slot_mapping entry differs from the slot the block table gives
 *                         the row's position (attention would read another row than the
 *                         append wrote)
 *   PA_CHECK_POSITION     with rotary_positions > 0: a new row's position is outside
 *                         [0, rotary_positions) (its cos/sin row does not exist)
 *   PA_CHECK_SLOT_DUP     two new rows would write the same cache slot (their slot_mapping
 *                         entries, or without slot_mapping the slots the block table gives their
 *                         positions; negative slots write nothing and do not count): the append
 *                         would race on that slot
 * slot_mapping may be NULL (not checked); block_table may be NULL (entries, and slot_mapping
 * against the table, not checked); rotary_positions = 0 skips the position rule.
 *   flags  int32 [1] (device), written by the call (cleared first); read it after the stream
 *          reaches the call. 0 means every rule holds.
 * Only the index arrays are read, inside their declared sizes; no index is followed, so any
 * contents are safe to check. Up to three launches (the duplicate-slot rule compares every pair
 * of new rows in 256-row tiles), no allocation, no host synchronisation.
 * Errors (besides these): PA_ERR_UNSUPPORTED when num_tokens needs more than 2^31 - 1 tile
 * pairs.
 * Errors: PA_ERR_NULL (shape, cumulative_sequence_length, past_seqlens or flags NULL),
 * PA_ERR_SHAPE or PA_ERR_UNSUPPORTED (the shape rules of pa_kv_append), PA_ERR_SHAPE
 * (rotary_positions < 0), PA_ERR_HIP.
 */
#define PA_CHECK_CU_START 1
#define PA_CHECK_CU_ORDER 2
#define PA_CHECK_CU_END 4
#define PA_CHECK_PAST 8
#define PA_CHECK_TABLE_WIDTH 16
#define PA_CHECK_TABLE_ENTRY 32
#define PA_CHECK_SLOT 64
#define PA_CHECK_SLOT_TABLE 128
#define PA_CHECK_POSITION 256
#define PA_CHECK_SLOT_DUP 512
pa_status pa_check_paged_indices(const pa_paged_shape *shape,
                                 const int32_t *cumulative_sequence_length,
                                 const int32_t *past_seqlens, const int32_t *block_table,
                                 const int32_t *slot_mapping, int32_t rotary_positions,
                                 int32_t *flags, void *stream);

/* Static description of a status code. */
const char *pa_status_string(pa_status status);

/*
 * Measurement hooks (not part of the computation). When enabled, every kernel the library
 * enqueues is bracketed by a pair of HIP events on its stream; pa_timing_get waits for the
 * recorded events and returns the summed milliseconds and the launch count of the kernels
 * whose name equals `kernel` (or of all kernels when kernel is NULL). pa_timing_reset drops
 * every record. Enabling timing adds two event records per launch.
 */
void pa_timing_enable(int32_t on);
void pa_timing_reset(void);
pa_status pa_timing_get(const char *kernel, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
