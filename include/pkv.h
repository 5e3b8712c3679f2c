/*
 * pkv.h - decode-step attention over a paged KV cache, for AMD MI355X (gfx950).
 *
 * One decode step: every sequence appends the K/V rows of its one new token,
 * then its new query attends over all of its cached tokens.  The cache of
 * every sequence lives in fixed-size physical blocks of a shared pool; a
 * per-sequence block table maps logical block j (tokens j*bs .. j*bs+bs-1) to
 * a physical block anywhere in the pool.
 *   - KV-cache post (xuewyang.github.io/posts/kv), "Prefill and decode" and
 *     "PagedAttention: the KV cache in blocks";
 *   - brunomaga.github.io inference post, "PagedAttention: memory management
 *     for the KV cache" (PagedKVCache, paged_decode_attention);
 *   - learn.mohebi.ai serving lesson, "PagedAttention" (block-by-block reads
 *     merged with the online-softmax update) and "Where it shows up"
 *     (split-KV decoding).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers marked [device] are device memory owned by the caller; the library
 * allocates nothing, keeps no state between calls and never synchronises the
 * host.  Every call enqueues its kernels on `stream` (a hipStream_t, passed as
 * void* so that this header needs no HIP header; NULL is the default stream)
 * and returns.  Calls on one stream run in order; calls
 * on different streams that touch the same memory race.
 *
 * Layouts (row-major, innermost last):
 *   pools        [num_blocks, num_kv_heads, block_size, head_dim]  kv dtype
 *   block_tables int32 [num_seqs, max_blocks_per_seq]; entries past a
 *                sequence's ceil(ctx/block_size) blocks are never read
 *   context_lens int32 [num_seqs]; ctx counts the token appended this step
 *   q, out       [num_seqs, num_q_heads, head_dim] (the [B, Hq, 1, D] query
 *                of one decode step with the length-1 axis dropped)
 *   k_new, v_new [num_seqs, num_kv_heads, head_dim] in the pool's dtype
 *   k_scales, v_scales float32 [num_blocks, num_kv_heads] (e4m3 pools only):
 *                stored value * scale = the real value
 * Query head i reads KV head i / (num_q_heads / num_kv_heads): consecutive
 * grouping, as in 32 query heads sharing 8 KV heads in groups of 4.
 *
 * Alignment: pools, q, out, k_new, v_new, partial outputs and the workspace
 * must be 16-byte aligned (the kernels move 16-byte vectors); int32 and
 * float32 arrays 4-byte aligned.  A misaligned pointer is PKV_ERR_INVALID_ARG.
 *
 * Device-side contract (not checked on the host, since the values live in
 * device memory): 0 <= ctx <= max_blocks_per_seq * block_size,
 * ctx <= max_context_len, and the first ceil(ctx/block_size) table entries of
 * each sequence are in [0, num_blocks).  The kernels never read or write
 * outside the buffers described here even when it is violated: a table entry
 * outside [0, num_blocks) is treated as an empty block, ctx is clamped to
 * the table's capacity, and tokens past max_context_len are ignored (fixed
 * partitions; the balanced split sizes nothing by max_context_len and attends
 * up to the clamped ctx).  Results are then unspecified, but no fault
 * follows.
 *
 * Errors are returned as pkv_status_t; nothing is launched when a call
 * returns anything but PKV_OK, except PKV_ERR_HIP (a launch failed).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

typedef enum {
  PKV_F32 = 0,       /* IEEE binary32                                        */
  PKV_BF16 = 1,      /* bfloat16 (top half of a binary32)                    */
  PKV_FP8_E4M3 = 2   /* OCP float8 e4m3fn: bias 7, max 448, no inf, NaN=0x7F */
} pkv_dtype_t;

/* Scale policy of pkv_kv_append_quant. */
typedef enum {
  PKV_SCALE_FIXED = 0,        /* keep each (block, head) scale as allocated          */
  PKV_SCALE_RUNNING_AMAX = 1  /* grow it to cover the new rows, requantising the block */
} pkv_scale_mode_t;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad relation */
  PKV_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim, block_size, dtypes */
  PKV_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  PKV_ERR_HIP = 4,           /* a HIP launch failed */
  PKV_ERR_OUT_OF_BLOCKS = 5  /* the block allocator has too few free blocks; nothing changed */
} pkv_status_t;

/* The version of this header the library was built from (PKV_ABI_VERSION). */
int pkv_abi_version(void);

/* A static, human-readable name for a status code. */
const char* pkv_status_string(pkv_status_t status);

/*
 * pkv_kv_append - write each sequence's new K and V rows into its slot.
 *
 * For every sequence b with ctx_b = context_lens[b] >= 1: position
 * pos = ctx_b - 1, physical block blk = block_tables[b][pos / block_size],
 * slot off = pos % block_size; then for every KV head h,
 * k_pool[blk][h][off][:] = k_new[b][h][:] and likewise for V.  A bitwise
 * copy: e4m3 rows arrive already quantised with the block's scale.  The block
 * must already be in the table (allocation is the caller's job; the pages'
 * PagedKVCache.append takes a new block when pos % block_size == 0).  A
 * sequence with ctx_b <= 0 is skipped.  Nothing else in the pools changes.
 *   KV-cache post, "A toy vLLM" (write_kv) and "Reading the code";
 *   brunomaga inference post, "PagedAttention..." (PagedKVCache.append).
 *
 * k_pool, v_pool [device, written]; k_new, v_new, block_tables, context_lens
 * [device, read].  Sizes as in the header comment.  num_seqs == 0 is a no-op.
 * Supported: head_dim in {64, 128}, block_size == 16, kv_dtype any.
 */
pkv_status_t pkv_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, pkv_dtype_t kv_dtype, void* stream);

/*
 * partition_size asking for a balanced split (pkv_paged_decode_attention,
 * pkv_paged_decode_step, pkv_mla_decode_attention and their workspace
 * sizes).  Instead of fixed partitions, each sequence's blocks (pairs of
 * blocks for MLA) are divided into n_b >= 1 chunks of nearly equal size,
 * n_b = max(1, ceil(u_b / t)) for its u_b units, with t the smallest chunk
 * size for which the batch needs at most R chunks.  S, the chunk slots of
 * one wave of workgroups MI355X runs at once, sets R: one-token decode,
 * S = 3072 / (num_kv_heads x column tiles) and R = S when 2 num_seqs <= S,
 * else max(2 S, 2 num_seqs) (pkv_decode_plan_slots); MLA, S = 256 for more
 * than 64 heads, 512 otherwise, and R = max(S, num_seqs).  The schedule is
 * computed on the device from context_lens (no host copy, so a call stays
 * capturable in a graph): for up to 256 sequences each decode workgroup
 * derives it itself, otherwise a one-wave kernel runs first.  The chunks are
 * run and merged; a sequence with one chunk is written directly.  The result
 * equals a fixed-partition split's up to float
 * rounding: only the grouping of the partial sums changes (the log-sum-exp
 * merge combines any split of the tokens).  Intended for batches of uneven or
 * long contexts, where a fixed partition size leaves the kernel waiting for
 * its longest partitions.
 * max_context_len is not used to size anything in this mode.
 *   serving lesson, "Where it shows up" (split-KV decoding spreads one
 *   sequence over the whole GPU).
 */
#define PKV_PARTITION_BALANCED (-1)

/*
 * pkv_decode_workspace_bytes - device workspace that
 * pkv_paged_decode_attention needs for its split-KV partial results:
 * float32 o [num_seqs, num_q_heads, maxP, head_dim] then, at the next
 * 256-byte boundary, float32 lse [num_seqs, num_q_heads, maxP], where
 * maxP = ceil(max_context_len / partition_size) (1 when partition_size == 0).
 * Returns 0 when maxP <= 1 (no workspace is needed) or on invalid sizes.
 * With PKV_PARTITION_BALANCED: float32 o [R, num_q_heads, head_dim], float32
 * lse [R, num_q_heads] and the plan of pkv_decode_plan for R slots, each
 * 256-byte aligned, for R = max(2 x 3072 / ceil(num_q_heads / 16),
 * 2 num_seqs), an upper bound of the slots a call uses (the call itself needs
 * them for R = pkv_decode_plan_slots(...) only).
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size);

/*
 * pkv_paged_decode_attention - one query token per sequence attends over its
 * whole paged cache (call pkv_kv_append first, on the same stream).
 *
 * out[b][i][:] = sum_t p_t * V[b][h][t][:],  p = softmax_t(softmax_scale *
 * q[b][i] . K[b][h][t]),  h = i / (num_q_heads / num_kv_heads),  over the
 * tokens t < ctx_b gathered through the block table; no other mask.  For
 * e4m3 pools K and V are scaled by their (block, head) scale.  Scores, the
 * softmax, sums and accumulators are float32; with bf16 queries over a bf16
 * cache and 2 or more query heads per KV head the product P.V runs on the
 * matrix cores with the weights P rounded to bfloat16 (relative error at most
 * 2^-9 per weight).  out is written in q_dtype (bfloat16 rounded to nearest
 * even).  A sequence with ctx_b == 0 gets zeros.
 *   brunomaga inference post, paged_decode_attention (the definition);
 *   serving lesson, "PagedAttention" (block-by-block, online softmax) and
 *   "Where it shows up" (split-KV decoding over the whole GPU).
 *
 * The tokens of each sequence are split into partitions of partition_size
 * tokens (a multiple of block_size; 0 = one partition per sequence).  One
 * workgroup per (sequence, KV head, partition) streams the partition's blocks
 * once for all the query heads of its group and writes a normalised partial
 * output plus its natural-log log-sum-exp to `workspace`; a second kernel
 * merges them (skipped when maxP == 1, where the first writes `out`).
 * partition_size == PKV_PARTITION_BALANCED uses balanced chunks instead.
 *
 * out [device, written]; q, pools, scales, tables, lens [device, read];
 * workspace [device, scratch] of at least pkv_decode_workspace_bytes(...)
 * bytes (may be NULL when that is 0).  max_context_len: a host-side upper
 * bound of context_lens, used to size the grid.
 * Supported: head_dim in {64, 128}; block_size == 16; any
 * num_q_heads / num_kv_heads ratio; (q, kv) dtypes: q in {F32, BF16} with kv
 * in {F32, BF16, FP8_E4M3}; e4m3 needs k_scales and v_scales.
 */
pkv_status_t pkv_paged_decode_attention(
    void* out, const void* q, const void* k_pool, const void* v_pool,
    const float* k_scales, const float* v_scales, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float softmax_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream);

/*
 * pkv_paged_decode_step - one whole decode step: exactly pkv_kv_append
 * followed by pkv_paged_decode_attention, with the append done inside the
 * decode kernel.  The workgroup that reads a sequence's last block takes the
 * new token's K/V rows from k_new/v_new and writes them into their pool slot
 * (slot ctx-1, bit for bit), so the step costs one decode launch (plus the
 * merge) instead of a separate append launch.  Pools and outputs afterwards
 * are those of the two separate calls.
 *   KV-cache post, "Prefill and decode": the token's own K/V are appended
 *   first, then everything cached is attended.
 *
 * Arguments as for pkv_kv_append and pkv_paged_decode_attention; k_pool and
 * v_pool are [device, read and written].  The append of a sequence happens
 * only if 1 <= ctx <= max_blocks_per_seq * block_size and (fixed
 * partitions) ctx <= max_context_len (the launched partitions cover its last
 * block; balanced chunks always cover it).
 */
pkv_status_t pkv_paged_decode_step(
    void* out, const void* q, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
    const float* k_scales, const float* v_scales, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float softmax_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream);

/*
 * pkv_paged_decode_step_noalloc - pkv_paged_decode_step without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The split-KV partial results (and the balanced split's plan) go to a
 * device array inside the library, PKV_NOALLOC_SCRATCH_BYTES bytes on each
 * GPU it runs on, held until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the first call on a
 * device looks the array's address up with that device current.  Same
 * arguments, kernels and results as pkv_paged_decode_step with a caller
 * workspace.  Returns PKV_ERR_WORKSPACE, and launches nothing, when the call
 * needs more than PKV_NOALLOC_SCRATCH_BYTES of workspace (the exact layout
 * of this call, at most pkv_decode_workspace_bytes(...); e.g. 6.3 MB for
 * batch 64 x 32 q heads x head dim 128 with PKV_PARTITION_BALANCED), and
 * PKV_ERR_HIP when the address lookup fails.  Every call on one GPU shares
 * that GPU's array and leaves its results there: calls that overlap on one
 * GPU (different streams, or different host threads without ordering) race
 * and give undefined results.  Nothing in the array needs to start at zero.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
pkv_status_t pkv_paged_decode_step_noalloc(
    void* out, const void* q, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
    const float* k_scales, const float* v_scales, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float softmax_scale, int32_t partition_size, pkv_dtype_t q_dtype,
    pkv_dtype_t kv_dtype, void* stream);

/*
 * pkv_paged_decode_partials - the split-KV half of pkv_paged_decode_attention
 * on its own: per-partition attention results, not merged.
 *
 * Partition p of sequence b covers its tokens [p*P, min((p+1)*P, ctx_b))
 * (P = partition_size; 0 means one partition holding the whole sequence).
 * For p < ceil(ctx_b / P) it writes the normalised partial output
 * partial_out[b][i][p][:] = sum_t p_t V_t / sum_t p_t over the partition's
 * tokens and partial_lse[b][i][p] = ln sum_t exp(s_t) (s_t the scaled scores,
 * natural log); for the partitions ceil(ctx_b / P) <= p < max_partitions it
 * writes partial_lse = -inf and leaves partial_out untouched.  Tokens at or
 * beyond max_partitions * P are not read.  pkv_merge_partials on the result
 * gives pkv_paged_decode_attention's output.  This is the piece each GPU runs
 * over its own token range when one sequence's cache is split across GPUs.
 *   serving lesson, "PagedAttention" and "Where it shows up" (partial results
 *   of split-KV decoding, merged afterwards).
 *
 * partial_out float32 [num_seqs, num_q_heads, max_partitions, head_dim] and
 * partial_lse float32 [num_seqs, num_q_heads, max_partitions] [device,
 * written]; the other arguments as for pkv_paged_decode_attention.
 */
pkv_status_t pkv_paged_decode_partials(
    float* partial_out, float* partial_lse, int32_t max_partitions, const void* q,
    const void* k_pool, const void* v_pool, const float* k_scales, const float* v_scales,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale, int32_t partition_size,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream);

/*
 * pkv_merge_partials - combine per-partition attention results.
 *
 * For each (b, i): M = max_p lse[b][i][p] over the partitions that count,
 * w_p = exp(lse_p - M), out[b][i][:] = sum_p w_p o[b][i][p][:] / sum_p w_p.
 * A partition counts if p < num_partitions[b] (all max_partitions when
 * num_partitions is NULL) and its lse is not -inf; partitions that do not
 * count are never multiplied (their o may hold anything).  With no counting
 * partition the output is 0.  lse is the natural log of the partition's
 * softmax denominator in the same units as its scores (m + ln sum exp(s - m)).
 *   serving lesson, "PagedAttention" / "Where it shows up": partial results
 *   of blocks or of a split cache merged by the online-softmax update.
 *
 * out [device, written] [num_seqs, num_q_heads, head_dim] in out_dtype
 * (F32 or BF16); partial_out float32 [num_seqs, num_q_heads, max_partitions,
 * head_dim] and partial_lse float32 [num_seqs, num_q_heads, max_partitions]
 * [device, read]; num_partitions int32 [num_seqs] [device, read] or NULL.
 * Supported: head_dim in {64, 128, 512} (512: MLA latent rows).
 */
pkv_status_t pkv_merge_partials(void* out, const float* partial_out, const float* partial_lse,
                                const int32_t* num_partitions, int32_t num_seqs,
                                int32_t num_q_heads, int32_t head_dim, int32_t max_partitions,
                                pkv_dtype_t out_dtype, void* stream);

/*
 * The balanced split in separate calls (the pieces of
 * pkv_paged_decode_attention with PKV_PARTITION_BALANCED, for callers that
 * reuse one schedule, time the pieces, or merge chunk results themselves).
 *
 * pkv_decode_plan_slots - R, the chunk slots of a balanced split for this
 * shape and dtype pair (the value the attention call uses, see
 * PKV_PARTITION_BALANCED); 0 for invalid arguments.
 *
 * pkv_decode_plan_bytes - bytes of a plan for num_seqs sequences and
 * num_slots slots: int32 chunk_first [num_seqs + 1], then, 256-byte aligned,
 * int32x4 slot_info [num_slots] = {sequence, first block, end block, chunks
 * of that sequence}, or {-1, 0, 0, 0} past the last chunk.  0 when num_slots
 * < max(1, num_seqs) or on invalid sizes.
 *
 * pkv_decode_plan - writes the plan [device, written, 16-byte aligned, at
 * least pkv_decode_plan_bytes] from context_lens [device, read]: sequence b
 * (its ctx clamped to [0, max_blocks_per_seq * block_size]) owns slots
 * chunk_first[b] .. chunk_first[b+1]-1, chunk k of its n_b covering blocks
 * [k u_b / n_b, (k+1) u_b / n_b) of its u_b = ceil(ctx / block_size); see
 * PKV_PARTITION_BALANCED for n_b (here R = max(num_slots, num_seqs)).
 *
 * pkv_paged_decode_partials_planned - the decode half of a balanced
 * attention call: it schedules the batch over num_slots slots (as
 * pkv_decode_plan does) and runs the chunks.  For slot s of sequence b it
 * writes the normalised partial output over the chunk's tokens to
 * partial_out[s][i][:] and its natural-log log-sum-exp to partial_lse[s][i]
 * (-inf for an empty sequence's one chunk); slots past the last chunk are not
 * written.  plan [device, written; plan_bytes >= pkv_decode_plan_bytes(
 * num_seqs, num_slots), else PKV_ERR_WORKSPACE] receives chunk_first (and,
 * for more than 256 sequences or 46,340 slots, slot_info: smaller batches are
 * scheduled inside the decode kernel itself, larger ones by a separate plan
 * kernel first).  partial_out float32 [num_slots, num_q_heads, head_dim],
 * partial_lse float32 [num_slots, num_q_heads] [device, written]; the rest as
 * for pkv_paged_decode_partials.
 *
 * pkv_merge_partials_planned - out[b][i][:] = the log-sum-exp merge (as
 * pkv_merge_partials) of rows chunk_first[b] .. chunk_first[b+1]-1 of
 * partial_out / partial_lse laid out as above; out in out_dtype (F32, BF16).
 *   serving lesson, "Where it shows up" (split-KV partial results merged).
 */
int32_t pkv_decode_plan_slots(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype);
size_t pkv_decode_plan_bytes(int32_t num_seqs, int32_t num_slots);
pkv_status_t pkv_decode_plan(void* plan, size_t plan_bytes, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_slots, int32_t block_size,
                             int32_t max_blocks_per_seq, void* stream);
pkv_status_t pkv_paged_decode_partials_planned(
    float* partial_out, float* partial_lse, void* plan, size_t plan_bytes, int32_t num_slots,
    const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales,
    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale, pkv_dtype_t q_dtype,
    pkv_dtype_t kv_dtype, void* stream);
pkv_status_t pkv_merge_partials_planned(void* out, const float* partial_out,
                                        const float* partial_lse, const void* plan,
                                        int32_t num_slots, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t head_dim, pkv_dtype_t out_dtype, void* stream);

/*
 * Several new tokens per sequence
 * -------------------------------
 * The entry points below serve a step in which sequence b brings t_b >= 0 new
 * tokens instead of one: a chunk of a long prompt (chunked prefill), the
 * uncached tail of a prompt whose prefix is cached, or draft tokens checked
 * in one pass.  Their rows are stacked over sequences:
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, query_start_loc[0]
 *                = 0 and query_start_loc[num_seqs] = num_tokens; rows
 *                query_start_loc[b] .. query_start_loc[b+1]-1 are sequence
 *                b's new tokens in order, t_b their count
 *   q, out       [num_tokens, num_q_heads, head_dim]
 *   k_new, v_new [num_tokens, num_kv_heads, head_dim] in the pool's dtype
 * context_lens[b] counts the t_b new tokens: they take positions
 * ctx_b - t_b .. ctx_b - 1.  Device-side contract, beyond the one above:
 * query_start_loc as described and t_b <= max_query_len.
 */

/*
 * pkv_kv_append_tokens - write each sequence's t_b new K and V rows into
 * their slots: row query_start_loc[b] + j goes to position ctx_b - t_b + j
 * (block block_tables[b][pos / block_size], slot pos % block_size), for every
 * KV head, bit for bit.  Rows whose position would be negative, and every row
 * of a sequence with ctx_b <= 0 or ctx_b past the table's capacity, are
 * skipped.  With t_b = 1 for all b this is pkv_kv_append.
 *   KV-cache post, "A KV cache in PyTorch" (the t new keys and values are
 *   concatenated after the cached ones); 4yush post, "Adding the cache to
 *   GPT-2" (new token r takes position start + r).
 *
 * k_pool, v_pool [device, written]; k_new, v_new, block_tables, context_lens,
 * query_start_loc [device, read].  num_tokens == 0 or num_seqs == 0 is a
 * no-op.  Supported as for pkv_kv_append.
 */
pkv_status_t pkv_kv_append_tokens(void* k_pool, void* v_pool, const void* k_new,
                                  const void* v_new, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* query_start_loc,
                                  int32_t num_seqs, int32_t num_tokens, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, pkv_dtype_t kv_dtype,
                                  void* stream);

/*
 * pkv_multi_query_workspace_bytes - device workspace of
 * pkv_paged_multi_query_attention: float32 o [num_tokens, num_q_heads, maxP,
 * head_dim] then, at the next 256-byte boundary, float32 lse [num_tokens,
 * num_q_heads, maxP], maxP = ceil(max_context_len / partition_size) (1 when
 * partition_size == 0).  Returns 0 when maxP <= 1 or on invalid sizes.
 */
size_t pkv_multi_query_workspace_bytes(int32_t num_tokens, int32_t num_q_heads,
                                       int32_t head_dim, int32_t max_context_len,
                                       int32_t partition_size);

/*
 * pkv_multi_query_balanced_workspace_bytes - device workspace of
 * pkv_paged_multi_query_attention with PKV_PARTITION_BALANCED (which
 * pkv_multi_query_workspace_bytes cannot size: it depends on the KV heads and
 * the longest query): float32 o [R, max_query_len, num_q_heads, head_dim],
 * float32 lse [R, max_query_len, num_q_heads] and a plan of
 * pkv_decode_plan_bytes(num_seqs, R) bytes, each 256-byte aligned, R the
 * chunk slots for num_kv_heads x ceil(max_query_len x group / tile) units
 * (as pkv_decode_plan_slots counts them for one new token).  0 on invalid
 * arguments.
 */
size_t pkv_multi_query_balanced_workspace_bytes(int32_t num_seqs, int32_t max_query_len,
                                                int32_t num_q_heads, int32_t num_kv_heads,
                                                int32_t head_dim, pkv_dtype_t q_dtype,
                                                pkv_dtype_t kv_dtype);

/*
 * pkv_paged_multi_query_attention - every new token attends over the cached
 * tokens up to and including its own position (call pkv_kv_append_tokens
 * first, on the same stream): the causal mask shifted by the cache length.
 *
 * For row r = query_start_loc[b] + j (0 <= j < t_b) and query head i:
 * out[r][i][:] = sum_{s < n} p_s V[b][h][s][:], p = softmax_s(softmax_scale *
 * q[r][i] . K[b][h][s]), h = i / (num_q_heads / num_kv_heads), over the
 * n = ctx_b - t_b + j + 1 tokens before and at its position.  A row with
 * n <= 0 gets zeros.  Precision and dtypes as for pkv_paged_decode_attention
 * (the matrix cores run bf16 over bf16 with 2 or more query heads per KV
 * head); with t_b = 1 for all b the result is that of
 * pkv_paged_decode_attention.
 *   KV-cache post, "A KV cache in PyTorch" (the mask tril(T - t) over the
 *   cached plus new keys); brunomaga inference post, causal_mask(Sq, Sk) =
 *   tril(Sk - Sq); 4yush post, "Adding the cache to GPT-2".
 *
 * One workgroup per (sequence, KV head, tile of query columns, partition):
 * column n of sequence b is new token n / g and head n % g of the KV head's
 * group (g = num_q_heads / num_kv_heads), so the g*t_b queries that share a
 * KV head read each cached block once per partition.  Partitions are merged
 * as in pkv_paged_decode_attention.  partition_size == PKV_PARTITION_BALANCED
 * splits each sequence's blocks into balanced chunks as for one new token
 * (every query of a chunk's sequence attends over the chunk; partial rows
 * [slot, max_query_len, num_q_heads]).
 *
 * out [device, written] in q_dtype; q, pools, scales, tables, lens,
 * query_start_loc [device, read]; workspace [device, scratch] of at least
 * pkv_multi_query_workspace_bytes(num_tokens, ...) bytes (may be NULL when
 * that is 0), or pkv_multi_query_balanced_workspace_bytes(...) bytes for the
 * balanced split.  max_query_len: a host-side upper bound of every t_b (>= 1),
 * used to size the grid; max_context_len as for pkv_paged_decode_attention.
 * Supported as for pkv_paged_decode_attention.
 */
pkv_status_t pkv_paged_multi_query_attention(
    void* out, const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
    float softmax_scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream);

/*
 * pkv_paged_multi_query_partials - the split-KV half of
 * pkv_paged_multi_query_attention on its own, as pkv_paged_decode_partials is
 * for one new token: for row r of sequence b, query head i and partition p <
 * ceil(ctx_b / P), the normalised partial output over the partition's tokens
 * that the row sees and its natural-log log-sum-exp (-inf when the row sees
 * none of them; partial_out then carries no meaning); partitions
 * ceil(ctx_b / P) <= p < max_partitions get lse = -inf and leave partial_out
 * untouched.  pkv_merge_partials
 * over the num_tokens rows gives pkv_paged_multi_query_attention's output.
 *
 * partial_out float32 [num_tokens, num_q_heads, max_partitions, head_dim] and
 * partial_lse float32 [num_tokens, num_q_heads, max_partitions] [device,
 * written]; the other arguments as for pkv_paged_multi_query_attention.
 */
pkv_status_t pkv_paged_multi_query_partials(
    float* partial_out, float* partial_lse, int32_t max_partitions, const void* q,
    const void* k_pool, const void* v_pool, const float* k_scales, const float* v_scales,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
    int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    int32_t max_blocks_per_seq, float softmax_scale, int32_t partition_size,
    pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype, void* stream);

/*
 * The balanced split with several new tokens per sequence, decode half alone
 * (what pkv_paged_multi_query_attention with PKV_PARTITION_BALANCED runs
 * before its merge; for callers that time the decode kernel or merge chunk
 * results themselves).
 *
 * pkv_multi_query_plan_slots - R, the chunk slots that call uses for this
 * shape, max_query_len and dtype pair (see PKV_PARTITION_BALANCED: S = 3072,
 * or 2048 when a wave holds two 16-column tiles, divided by num_kv_heads x
 * column chunks); 0 for invalid arguments.
 *
 * pkv_paged_multi_query_partials_planned - schedules the batch over
 * num_slots slots exactly as pkv_paged_decode_partials_planned does (plan
 * [device, written], its layout and the PKV_ERR_WORKSPACE rule as there) and
 * runs the chunks.  For slot s of sequence b and its new token j < t_b it
 * writes, for every query head i, the normalised partial output over the
 * chunk's tokens that token j sees (positions up to ctx_b - t_b + j) to
 * partial_out[s][j][i][:] and their natural-log log-sum-exp to
 * partial_lse[s][j][i] (-inf when it sees none of them; partial_out then
 * holds nothing meaningful); rows j >= t_b and slots past the last chunk are
 * not written.  The
 * log-sum-exp merge of a row over its sequence's slots chunk_first[b] ..
 * chunk_first[b+1]-1 gives pkv_paged_multi_query_attention's output.
 *   KV-cache post, "A KV cache in PyTorch" (the shifted causal mask of
 *   attn_cached); serving lesson, "Where it shows up" (split-KV decoding).
 *
 * partial_out float32 [num_slots, max_query_len, num_q_heads, head_dim] and
 * partial_lse float32 [num_slots, max_query_len, num_q_heads] [device,
 * written]; num_slots >= num_seqs; the rest as for
 * pkv_paged_multi_query_attention.
 */
int32_t pkv_multi_query_plan_slots(int32_t num_seqs, int32_t max_query_len,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   pkv_dtype_t q_dtype, pkv_dtype_t kv_dtype);
pkv_status_t pkv_paged_multi_query_partials_planned(
    float* partial_out, float* partial_lse, void* plan, size_t plan_bytes, int32_t num_slots,
    const void* q, const void* k_pool, const void* v_pool, const float* k_scales,
    const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale, pkv_dtype_t q_dtype,
    pkv_dtype_t kv_dtype, void* stream);

/*
 * pkv_kv_append_quant - append new K/V rows given in bf16 or float32 to an
 * e4m3 cache, quantising them with their (block, KV head) scale: the code of
 * a value x is encode(f32(x / s)), one correctly rounded float32 division
 * followed by rounding to the nearest e4m3fn value, ties to the even code,
 * saturating at +-448 (NaN gives 0x7F).  Placement is that of
 * pkv_kv_append_tokens (query_start_loc NULL: one row per sequence, row b
 * to position ctx_b - 1, as pkv_kv_append).
 *   KV-cache post, "The KV cache is big" (fewer bytes per number: an 8-bit
 *   cache halves it); serving lesson, "Smaller caches: GQA, MQA, MLA and
 *   quantized caches" (an fp8 cache halves e).
 *
 * mode PKV_SCALE_FIXED: every slice keeps the scale the caller gave its
 * block at allocation (k_scales/v_scales are only read); values beyond
 * 448 * s saturate.  mode PKV_SCALE_RUNNING_AMAX: for the new rows landing
 * in one slice, amax = max |x| and the slice's scale becomes
 * max(old, f32(amax / 448)), where old is ignored (taken as 0) if the first
 * new row sits at slot 0 (a fresh block).  If the scale grew and the slice
 * has earlier rows, each earlier code c is requantised to
 * encode(f32(f32(decode(c) * old) / new)).  A scale of 0 (all values so far
 * 0) stores code 0.  Scales never shrink.  The decode kernels read the
 * result as any e4m3 cache (value = code * scale).
 *
 * k_pool, v_pool [device, read and written] e4m3 codes [num_blocks,
 * num_kv_heads, block_size, head_dim]; k_scales, v_scales [device, read, and
 * written in running mode] float32 [num_blocks, num_kv_heads]; k_new, v_new
 * [device, read] [num_rows, num_kv_heads, head_dim] in new_dtype (F32 or
 * BF16); block_tables, context_lens, query_start_loc [device, read].  One
 * workgroup per (sequence, KV head) handles that sequence's slices in order,
 * so no two sequences may append into the same physical block (copy a shared
 * block first).  New rows must be finite.  num_seqs == 0 or num_rows == 0 is
 * a no-op.  Supported: head_dim in {64, 128}, block_size == 16.
 */
pkv_status_t pkv_kv_append_quant(void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                                 const void* k_new, const void* v_new, pkv_dtype_t new_dtype,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* query_start_loc, int32_t num_seqs,
                                 int32_t num_rows, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, pkv_scale_mode_t mode,
                                 void* stream);

/*
 * Block allocator (host side) and copy-on-write copies (device side)
 * ------------------------------------------------------------------
 * The memory manager just above the kernels.  Blocks are handed out on
 * demand: a sequence takes a new block only when its last one is full, so it
 * wastes at most block_size - 1 slots; a finished sequence returns its blocks
 * at once.  The free list starts as 0 .. num_blocks-1, allocation takes its
 * last entry and freeing appends the sequence's table in order.  A physical
 * block may be held by several sequences (forked samples of one prompt); a
 * reference count says how many.  Before a sequence writes into a block whose
 * count is above 1 it moves to a private copy: a fresh block, the old block's
 * count minus 1, and a (src, dst) pair for pkv_copy_blocks.  The last sharer
 * writes in place.  Only a partly filled last block is ever written, so one
 * append needs at most one copy.
 *   KV-cache post, "PagedAttention: the KV cache in blocks" (allocate on
 *   demand, free immediately, sharing with copy-on-write); brunomaga post,
 *   "PagedAttention: memory management for the KV cache" (PagedKVCache:
 *   free-list order, out of blocks is the scheduler's problem); serving
 *   lesson, "Sharing (section 4.4)" and exercise 3 (three samples of a
 *   100-token prompt: 21 blocks unshared, 7 shared, 9 after each writes one
 *   token).
 * The allocator is plain host memory, not thread-safe (one scheduler thread
 * owns it), and never touches the GPU.  Sequence ids are caller-chosen int64.
 */
typedef struct pkv_block_manager pkv_block_manager_t;

/* A new allocator over num_blocks blocks of block_size tokens; NULL on bad sizes or no memory. */
pkv_block_manager_t* pkv_bm_create(int32_t num_blocks, int32_t block_size);
void pkv_bm_destroy(pkv_block_manager_t* bm);

/* An empty sequence.  PKV_ERR_INVALID_ARG if the id is taken. */
pkv_status_t pkv_bm_add_seq(pkv_block_manager_t* bm, int64_t seq_id);

/* child shares all of parent's blocks (counts + 1) and its length.  The
 * parent must exist and the child must not. */
pkv_status_t pkv_bm_fork(pkv_block_manager_t* bm, int64_t parent, int64_t child);

/* Drop a sequence: each of its blocks' counts - 1; blocks reaching 0 go back
 * to the free list in table order. */
pkv_status_t pkv_bm_free_seq(pkv_block_manager_t* bm, int64_t seq_id);

/* Make room for num_tokens new tokens of seq_id (positions len .. len+n-1):
 * new blocks as needed and, if the partly filled last block is shared, a
 * private copy of it, returned as copy_src[0] -> copy_dst[0] with
 * *num_copies = 1 (else 0).  copy_src/copy_dst [host, written] need room for
 * max_copies >= 1 entries when a copy is needed (else PKV_ERR_INVALID_ARG).
 * PKV_ERR_OUT_OF_BLOCKS, with nothing changed, when too few blocks are
 * free.  The caller must run the copies (pkv_copy_blocks) before writing the
 * new tokens. */
pkv_status_t pkv_bm_append_slots(pkv_block_manager_t* bm, int64_t seq_id, int32_t num_tokens,
                                 int32_t* copy_src, int32_t* copy_dst, int32_t max_copies,
                                 int32_t* num_copies);

/* Free blocks (-1 for a NULL allocator). */
int32_t pkv_bm_num_free(const pkv_block_manager_t* bm);
/* Reference count of a block (-1 if out of range). */
int32_t pkv_bm_refcount(const pkv_block_manager_t* bm, int32_t block);
/* Tokens of a sequence (-1 if unknown). */
int64_t pkv_bm_seq_len(const pkv_block_manager_t* bm, int64_t seq_id);
/* The free list, next allocation last: writes up to max_entries into out
 * [host] (may be NULL) and returns its length. */
int32_t pkv_bm_free_list(const pkv_block_manager_t* bm, int32_t* out, int32_t max_entries);

/* The block tables and lengths of num_seqs sequences, in the layout the
 * attention calls take: block_tables int32 [num_seqs, max_blocks_per_seq]
 * (-1 past each table) and context_lens int32 [num_seqs] [host, written].
 * PKV_ERR_INVALID_ARG (nothing written) for an unknown id or a table longer
 * than max_blocks_per_seq. */
pkv_status_t pkv_bm_block_tables(const pkv_block_manager_t* bm, const int64_t* seq_ids,
                                 int32_t num_seqs, int32_t* block_tables,
                                 int32_t max_blocks_per_seq, int32_t* context_lens);

/*
 * pkv_copy_blocks - run copy-on-write copies on the GPU: for each pair
 * (src, dst) of pairs int32 [num_pairs][2] [device, read], block dst of
 * k_pool and of v_pool (all num_kv_heads x block_size x head_dim elements)
 * becomes a bitwise copy of block src; for an e4m3 cache k_scales/v_scales
 * [device, read and written] rows dst become copies of rows src (the scales
 * are ignored, and may be NULL, for other dtypes).  Every copy reads the
 * state before the call: destinations must be distinct and none may be a
 * source.  Pairs with an id outside [0, num_blocks) are skipped.
 * Supported: head_dim in {64, 128}, block_size == 16, num_kv_heads <= 256.
 */
pkv_status_t pkv_copy_blocks(void* k_pool, void* v_pool, float* k_scales, float* v_scales,
                             const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             pkv_dtype_t kv_dtype, void* stream);

/*
 * Measurement: attainable read bandwidth
 * --------------------------------------
 * A decode step is left of the ridge point, where memory bandwidth is the
 * only roof (brunomaga inference post, "Roofline model"); what a kernel can
 * reach in practice is below the data-sheet peak.  pkv_stream_read does
 * nothing but read, so its rate over a buffer far larger than the last-level
 * cache is the practical read ceiling against which a decode kernel's rate
 * is judged.  Not part of the attention path.
 */
#define PKV_STREAM_READ_MAX_WORKGROUPS (1 << 20)

/* pkv_stream_read - read bytes of src [device, read; 16-byte aligned; bytes
 * a multiple of 16, may be 0] once, with 16-byte nontemporal loads, in
 * num_workgroups workgroups of 256 threads (1 .. PKV_STREAM_READ_MAX_WORKGROUPS)
 * striding over the buffer, and fold every 32-bit word read with XOR: out
 * uint32 [pkv_stream_read_out_words(num_workgroups)] [device, written] gets
 * one fold per wave, and the XOR of all of out is the XOR of all 32-bit
 * words of src.  PKV_ERR_INVALID_ARG for a bad count, size or pointer. */
pkv_status_t pkv_stream_read(uint32_t* out, const void* src, size_t bytes,
                             int32_t num_workgroups, void* stream);

/* pkv_gather_read - the same folded read over scattered 4 KiB chunks, the
 * unit a decode workgroup reads (one block of 16 tokens x 128 dims of one KV
 * head in bf16, anywhere in the pool): the practical read ceiling of that
 * access pattern.  src [device, read; 16-byte aligned] is bytes long, a
 * multiple of 4096; chunk_ids int32 [num_chunks] [device, read] lists chunk
 * c = bytes [4096 c, 4096 c + 4096); ids outside [0, bytes / 4096) read
 * nothing.  One-wave workgroups take chunks_per_workgroup consecutive
 * entries each (num_chunks a multiple of it, at most
 * PKV_STREAM_READ_MAX_WORKGROUPS workgroups), two chunks in registers, 16
 * bytes per lane and load; out uint32 [64 x num_chunks /
 * chunks_per_workgroup] [device, written]: lane l of workgroup w writes
 * out[64 w + l], the XOR of the 32-bit words it read.
 * PKV_ERR_INVALID_ARG for a bad count, size or pointer. */
pkv_status_t pkv_gather_read(uint32_t* out, const void* src, size_t bytes,
                             const int32_t* chunk_ids, int32_t num_chunks,
                             int32_t chunks_per_workgroup, void* stream);

/* Words pkv_stream_read writes for num_workgroups workgroups (one per wave);
 * 0 for a count outside 1 .. PKV_STREAM_READ_MAX_WORKGROUPS. */
int32_t pkv_stream_read_out_words(int32_t num_workgroups);

/*
 * Multi-head latent attention (MLA), absorbed decode
 * --------------------------------------------------
 * An MLA layer caches one row per token: the latent c (kv_lora_rank = 512
 * numbers) followed by the rotary key shared by all heads (rope_dim = 64):
 * 576 numbers, against 2 x 128 x 128 for standard multi-head attention.
 * In decode the up-projections are folded away: the caller forms each
 * head's absorbed query [W_UK,i^T q_nope,i ; q_rope,i] (576 numbers), every
 * head attends over the shared rows directly (key = the whole row, value =
 * its latent), and the caller applies W_UV,i to the latent output.
 *   KV-cache post, "MLA: how does decode get full-size keys and values
 *   back?" (expand vs absorb; 512 + 64 numbers per token); serving lesson,
 *   "Smaller caches: GQA, MQA, MLA and quantized caches".
 * Layouts: latent_pool bf16 [num_blocks, block_size, 576]; block tables and
 * context_lens as above (ctx counts the appended token); q bf16 [num_seqs,
 * num_heads, 576]; out bf16 [num_seqs, num_heads, 512].
 */

/* pkv_mla_append - write each sequence's new 576-number row (latent_new bf16
 * [num_seqs, 576] [device, read]) into slot ctx-1 of latent_pool [device,
 * written], bit for bit; as pkv_kv_append with one shared head.  Supported:
 * row_dim == 576, block_size == 16. */
pkv_status_t pkv_mla_append(void* latent_pool, const void* latent_new,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t row_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq, void* stream);

/* Workspace of pkv_mla_decode_attention: float32 o [num_seqs, num_heads,
 * maxP, kv_lora_rank] then, 256-byte aligned, float32 lse [num_seqs,
 * num_heads, maxP]; 0 when maxP <= 1.  With PKV_PARTITION_BALANCED: o [R,
 * num_heads, kv_lora_rank] as bf16 (round to nearest even, in a region sized
 * for float32), float32 lse [R, num_heads] and int32 chunk starts
 * [num_seqs + 1], each 256-byte aligned, R = max(S, num_seqs)
 * (see PKV_PARTITION_BALANCED); max_context_len is not used.  0 for invalid
 * arguments. */
size_t pkv_mla_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t kv_lora_rank,
                               int32_t max_context_len, int32_t partition_size);

/*
 * pkv_mla_decode_attention - out[b][i][:] = sum_t p_t row_t[:512] with
 * p = softmax_t(softmax_scale * q[b][i] . row_t) over the ctx_b cached rows
 * of sequence b (no other mask).  Scores, softmax and sums are float32 on the
 * matrix cores with bf16 operands (the weights p rounded to bf16 for the
 * weighted sum); out is rounded to bf16.  A sequence with ctx 0 gets zeros.
 * Split-KV partitions of partition_size tokens are merged as in
 * pkv_paged_decode_attention; partition_size == PKV_PARTITION_BALANCED splits
 * the work into balanced chunks instead (three kernels: the split schedule,
 * the chunks, the merge; sequences that get one chunk are written directly).
 * One workgroup serves up to 128 heads, so each cached row is read from HBM
 * once per partition or chunk for all of them.
 * out [device, written]; q, latent_pool, tables, lens [device, read];
 * workspace [device, scratch] of pkv_mla_workspace_bytes(...) bytes.
 * Supported: kv_lora_rank == 512, rope_dim == 64, num_heads a multiple of
 * 16, block_size == 16, bf16.
 */
pkv_status_t pkv_mla_decode_attention(
    void* out, const void* q, const void* latent_pool, const int32_t* block_tables,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t kv_lora_rank,
    int32_t rope_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float softmax_scale, int32_t partition_size, void* workspace,
    size_t workspace_bytes, void* stream);

/* pkv_mla_decode_partials - the split-KV half of pkv_mla_decode_attention on
 * its own, as pkv_paged_decode_partials is for standard attention:
 * partial_out float32 [num_seqs, num_heads, max_partitions, 512] and
 * partial_lse float32 [num_seqs, num_heads, max_partitions] [device,
 * written]; partitions at or past ceil(ctx_b / P) get lse = -inf and leave
 * partial_out untouched.  pkv_merge_partials (head_dim 512, out bf16) gives
 * pkv_mla_decode_attention's output.  partition_size >= 0 only (the balanced
 * split's partials are grouped by chunk, not by partition). */
pkv_status_t pkv_mla_decode_partials(
    float* partial_out, float* partial_lse, int32_t max_partitions, const void* q,
    const void* latent_pool, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t kv_lora_rank, int32_t rope_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, float softmax_scale,
    int32_t partition_size, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
