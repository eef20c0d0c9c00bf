/*
 * pa.h -- paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Two operations, both defined by the
 * three web pages on paged KV caches this library follows:
 *
 *   [nano-vllm blog]  2kiu.com/news/6344849 -- "PagedAttention and prefix
 *                     caching", reproduced with nano-vllm (sections 1-7)
 *   [vLLM notes]      "vLLM: PagedAttention 与前缀缓存" (personal-site-7tw.pages.dev)
 *   [CANN notes]      discosf.com/news/6244710 -- Paged KV Cache and Packed
 *                     Sequence in cann-recipes-infer (sections 1-6)
 *
 * Data layout shared by both calls (all tensors contiguous, row-major):
 *   kv_pool       [num_blocks, 2, block_size, num_kv_heads, head_dim]
 *                 index 1 is 0 for K, 1 for V        ([CANN notes §2.1])
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; entry j of row s is
 *                 the physical block holding logical block j of sequence s
 *                 ([nano-vllm blog §2.2], [CANN notes §2.2]); entries past
 *                 ceil(len / block_size) are never read
 *   context_lens  int32 [num_seqs]: tokens in each sequence
 *   Token t of sequence s lives in block block_tables[s][t / block_size] at
 *   offset t % block_size ([CANN notes §2.2]).
 *
 * Element types (pa_dtype):
 *   PA_F16       IEEE binary16
 *   PA_BF16      bfloat16
 *   PA_FP8_E4M3  OCP fp8 E4M3 (bias 7, max 448, no infinities, 0x7F/0xFF NaN);
 *                a stored code c stands for value(c) * scale, with one fp32
 *                scale for all of K (k_scale) and one for all of V (v_scale).
 *                ([nano-vllm blog §1.1, §6.3] name fp8 KV; the encoding is
 *                the OCP one.)
 *
 * Pointers: every pointer is device memory owned by the caller, 16-byte
 * aligned, and stays valid until the work enqueued on `stream` completes.
 * The library allocates nothing and keeps no per-call state.  `stream` is a
 * hipStream_t (NULL = the default stream); every call only enqueues work on
 * it and returns without waiting.
 *
 * Errors: each call checks its arguments on the host before enqueueing
 * anything and returns a status; nothing is thrown across the ABI.  What the
 * host cannot check is the caller's contract: block-table entries that are
 * read must lie in [0, num_blocks), lengths must not exceed
 * max_blocks_per_seq * block_size, write slots must be distinct, and no write
 * may target a block that another table also references (shared blocks are
 * read-only, [nano-vllm blog §4.3]).  The kernels do not fault on a broken
 * contract: a block id outside the pool is skipped (its tokens are left out
 * of attention, its write is dropped) and a longer length is cut to
 * max_blocks_per_seq * block_size -- the results are then meaningless, but
 * memory outside the arguments is never touched.
 *
 * Size limit: one K (or V) half of a block, block_size * num_kv_heads *
 * head_dim elements, must stay below 4 GiB (else PA_ERR_BAD_SHAPE).
 *
 * Supported: head_dim 64 or 128; block_size 8, 16 or 32; num_heads a multiple
 * of num_kv_heads with num_heads / num_kv_heads in {1, 2, 4, 8} (query head h
 * reads KV head h / (num_heads / num_kv_heads)); (query, kv) dtypes
 * (F16, F16), (BF16, BF16) and (BF16, FP8_E4M3).  Other combinations return
 * PA_ERR_UNSUPPORTED.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL                     */
    PA_ERR_BAD_SHAPE = 2,           /* a size is out of range or inconsistent         */
    PA_ERR_BAD_DTYPE = 3,           /* a dtype value is not a pa_dtype                */
    PA_ERR_UNSUPPORTED = 4,         /* valid but not implemented combination          */
    PA_ERR_MISALIGNED = 5,          /* a pointer is not 16-byte aligned               */
    PA_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes < pa_decode_workspace_size()   */
    PA_ERR_HIP = 7,                 /* the HIP runtime rejected a launch              */
    PA_ERR_POOL_EXHAUSTED = 8,      /* block manager: not enough free blocks          */
    PA_ERR_UNKNOWN_SEQUENCE = 9     /* block manager: no sequence with that id        */
} pa_status;

typedef enum pa_dtype {
    PA_F16 = 0,
    PA_BF16 = 1,
    PA_FP8_E4M3 = 2
} pa_dtype;

/*
 * pa_cache_write -- store each sequence's newest token into the paged pool
 * (the per-token KV write of [nano-vllm blog §4.1 step 3] and
 * [CANN notes §4.3 steps 1-3], vLLM's reshape_and_cache).
 *
 * For every sequence s with L = context_lens[s] > 0 (the length AFTER the new
 * token was appended), with t = L - 1, b = block_tables[s][t / block_size],
 * o = t % block_size:
 *     kv_pool[b][0][o][g][:] = enc(key[s][g][:])
 *     kv_pool[b][1][o][g][:] = enc(value[s][g][:])      for every KV head g
 * enc is a bit copy when src_dtype == kv_dtype; for PA_FP8_E4M3 it is
 * e4m3(float32(x) / k_scale) (v_scale for V): IEEE float32 division, round
 * to nearest with ties to even, magnitudes beyond 448 saturate to 448, NaN
 * stays NaN.  A sequence with context_lens[s] <= 0 writes nothing.  The block
 * holding slot t must already be in the table: allocating it when the tail
 * block is full is the host's job ([CANN notes §2.3], [nano-vllm blog §2.2]).
 *
 *   kv_pool       in/out  [num_blocks, 2, block_size, num_kv_heads, head_dim] of kv_dtype
 *   key, value    in      [num_seqs, num_kv_heads, head_dim] of src_dtype
 *   (src, kv) dtypes: (F16, F16), (BF16, BF16), (BF16, FP8_E4M3), (F16, FP8_E4M3)
 *   k_scale, v_scale      used only for FP8_E4M3; must then be finite and > 0
 */
pa_status pa_cache_write(void* kv_pool, pa_dtype kv_dtype,
                         const void* key, const void* value, pa_dtype src_dtype,
                         const int32_t* block_tables, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                         float k_scale, float v_scale, void* stream);

/*
 * pa_decode_partition_size -- how pa_decode splits sequences for split-K with
 * these arguments.  A positive `requested` (a multiple of block_size) is a
 * fixed partition: every sequence is cut into pieces of that many tokens,
 * and that value is returned.  `requested` 0 leaves the split to the
 * library: the batch's tokens, laid end to end (each sequence padded to
 * whole blocks), are cut on the device, per call, into equal chunks, one per
 * workgroup the GPU holds at once, so every compute unit is dealt the same
 * number of tokens; a chunk may span several sequences.  The return value is
 * then the shortest chunk the library uses.  Returns 0 for invalid
 * arguments.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, pa_dtype kv_dtype,
                                 int32_t requested);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs with
 * the same arguments (same `partition_size`) on the current device.  Returns
 * 0 for invalid arguments.  The workspace holds the partial results of the
 * split-K pieces and, with partition_size 0, where each sequence's pieces
 * lie.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                int32_t max_blocks_per_seq, pa_dtype kv_dtype,
                                int32_t partition_size);

/*
 * pa_decode -- one decode step of paged attention ([nano-vllm blog §2.3],
 * [CANN notes §4.3 step 4]).  For each sequence s with L = context_lens[s]
 * and each query head h, with g = h / (num_heads / num_kv_heads):
 *     z_t   = scale * k_scale * <query[s][h], K_t[g]>      t = 0 .. L-1
 *     p     = softmax(z)
 *     out[s][h] = v_scale * sum_t p_t * V_t[g]
 * where K_t / V_t are read through the block table; slots of the last block
 * at or beyond L are excluded (the tail mask of [nano-vllm blog §2.3]).  A
 * sequence with L <= 0 gets a zero output.  k_scale / v_scale apply to
 * FP8_E4M3 KV only (pass 1 otherwise).  The result is rounded to q_dtype
 * (nearest, ties to even) from float32 accumulation.
 *
 *   out           out     [num_seqs, num_heads, head_dim] of q_dtype
 *   query         in      [num_seqs, num_heads, head_dim] of q_dtype
 *   kv_pool       in      [num_blocks, 2, block_size, num_kv_heads, head_dim] of kv_dtype
 *   partition_size        0 = library choice (equal token chunks across the batch, see
 *                         pa_decode_partition_size), else a positive multiple of
 *                         block_size: tokens per split-K partition (a sequence shorter
 *                         than one partition is not split)
 *   workspace     scratch device memory of at least pa_decode_workspace_size(...) bytes
 *                         for per-partition partial results.  Its contents on entry do not
 *                         matter.  Calls that may run concurrently need separate workspaces.
 *
 * Two kernels on `stream`: workgroups of the first own a group of KV heads
 * and a token range (one partition of one sequence, or one chunk of the
 * batch) and write, for each sequence range they cover, either the final
 * output (the sequence's whole range) or a partial softmax state; the second
 * merges the partials of split sequences.  Output does not depend on which
 * physical blocks the table names, only on their logical order.
 */
pa_status pa_decode(void* out, const void* query, pa_dtype q_dtype,
                    const void* kv_pool, pa_dtype kv_dtype,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                    float scale, float k_scale, float v_scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partials, pa_decode_merge -- the two launches pa_decode makes, for
 * callers that want to schedule or time them separately.  Arguments and
 * checks are exactly those of pa_decode.  pa_decode_partials runs the
 * attention pass: it writes the final output of every sequence that fits in
 * one partition and leaves per-partition partial softmax states (running
 * max, sum, unnormalised output) in the workspace for the others.
 * pa_decode_merge, enqueued after it on the same stream with the same
 * arguments and workspace, combines those partials into the output of the
 * split sequences (split-K merge); it enqueues nothing when no sequence can
 * be split.  pa_decode == pa_decode_partials followed by pa_decode_merge.
 */
pa_status pa_decode_partials(void* out, const void* query, pa_dtype q_dtype,
                             const void* kv_pool, pa_dtype kv_dtype,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int32_t num_blocks, float scale, float k_scale, float v_scale,
                             int32_t partition_size, void* workspace, size_t workspace_bytes,
                             void* stream);
pa_status pa_decode_merge(void* out, const void* query, pa_dtype q_dtype,
                          const void* kv_pool, pa_dtype kv_dtype,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t num_blocks, float scale, float k_scale, float v_scale,
                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * pa_decode_write, pa_decode_write_partials -- pa_cache_write and pa_decode
 * (or pa_decode_partials) in one attention pass: the decode step of
 * [CANN notes §4.3] (write the new token, then read every block) with one
 * launch less.  The wave that reads the newest token (position L - 1) of a
 * sequence and KV head first stores that token's K and V rows, exactly as
 * pa_cache_write would (fp8: divided by k_scale / v_scale in IEEE fp32,
 * e4m3 round-to-nearest-even, saturating), then reads them back.
 *
 *   key, value   [num_seqs, num_kv_heads, head_dim] of src_dtype, which must
 *                equal q_dtype (else PA_ERR_UNSUPPORTED); 16-byte aligned.
 *   The other arguments, the workspace and the results are those of
 *   pa_decode / pa_decode_partials; pa_decode_merge completes
 *   pa_decode_write_partials.  Sequences with context_lens[s] <= 0, or
 *   longer than the table holds, are not written.  The pool afterwards is
 *   bit for bit what pa_cache_write leaves.
 */
pa_status pa_decode_write(void* out, const void* query, pa_dtype q_dtype,
                          const void* kv_pool, pa_dtype kv_dtype,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t num_blocks, float scale, float k_scale, float v_scale,
                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                          void* stream, const void* key, const void* value, pa_dtype src_dtype);
pa_status pa_decode_write_partials(void* out, const void* query, pa_dtype q_dtype,
                                   const void* kv_pool, pa_dtype kv_dtype,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                   int32_t num_blocks, float scale, float k_scale, float v_scale,
                                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                                   void* stream, const void* key, const void* value, pa_dtype src_dtype);

/*
 * pa_decode_shared, pa_decode_write_partials_shared -- pa_decode and
 * pa_decode_write_partials for batches whose sequences share prefix blocks
 * in aligned runs ([nano-vllm blog §3, §4.3]: prefix caching and fork map
 * several sequences' leading logical blocks to one physical block).
 *
 *   run_size   1 (no runs: exactly pa_decode / pa_decode_write_partials), 2,
 *              4 or 8 (else PA_ERR_UNSUPPORTED; < 1: PA_ERR_BAD_SHAPE).
 *              Sequences run_size*k .. run_size*k + run_size - 1 form run
 *              k; a trailing incomplete run has no shared partitions.
 *
 * A split-K partition that every sequence of a run holds whole, with at
 * least one token after it, and whose blocks the run's tables map to the
 * same physical blocks, is computed once for the run: one pass reads each
 * K/V row once and keeps a softmax state per sequence.  The table contents
 * decide this on the device, so any run_size gives the same results up to
 * float rounding order -- runs that share nothing cost only the check.  The
 * run form applies where num_heads == num_kv_heads (the vector kernel);
 * otherwise run_size is checked and ignored.  Arguments, workspace (sized by
 * pa_decode_workspace_size), results and errors are otherwise those of
 * pa_decode / pa_decode_write_partials, and pa_decode_merge completes
 * pa_decode_write_partials_shared.
 */
pa_status pa_decode_shared(void* out, const void* query, pa_dtype q_dtype,
                           const void* kv_pool, pa_dtype kv_dtype,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t num_blocks, float scale, float k_scale, float v_scale,
                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                           void* stream, int32_t run_size);
pa_status pa_decode_write_partials_shared(void* out, const void* query, pa_dtype q_dtype,
                                          const void* kv_pool, pa_dtype kv_dtype,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                          int32_t num_blocks, float scale, float k_scale, float v_scale,
                                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                                          void* stream, const void* key, const void* value, pa_dtype src_dtype,
                                          int32_t run_size);

/*
 * pa_cache_write_tokens -- the prompt-stage write: put a packed run of new
 * tokens per sequence into the pool ([CANN notes §3.1] packed layout,
 * [CANN notes §4.2] prompt write into block offsets; [nano-vllm blog §4.3]
 * only the uncached tail of a prompt is written).
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim] of src_dtype; the new
 *                 tokens of sequence s are rows cu_seqlens[s] ..
 *                 cu_seqlens[s+1]-1, in order.
 *   cu_seqlens    device int32 [num_seqs + 1], non-decreasing, from 0;
 *                 n_s = cu_seqlens[s+1] - cu_seqlens[s].
 *   context_lens  lengths AFTER the append: row i of sequence s is written at
 *                 position L_s - n_s + i (block block_tables[s][t / bs],
 *                 offset t % bs).  Rows with a negative position, rows past
 *                 cu_seqlens[num_seqs] and table entries outside the pool
 *                 are skipped.
 * Everything else (dtypes, fp8 encoding, shapes, alignment, errors) is as in
 * pa_cache_write, which is this call with one new token per sequence.
 */
pa_status pa_cache_write_tokens(void* kv_pool, pa_dtype kv_dtype, const void* key, const void* value,
                                pa_dtype src_dtype, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                float k_scale, float v_scale, void* stream);

/*
 * pa_prefill -- causal attention of packed new queries over the paged pool
 * ([CANN notes §3.1-3.3]: cu_seqlens bounds each sequence, queries see only
 * their own sequence and only keys not after their own position, K/V are
 * found through the block table; [nano-vllm blog §4.3]: the tail of a
 * prompt whose prefix is cached attends to that prefix too).
 *
 *   out, query    [num_tokens, num_heads, head_dim] of q_dtype (out may not
 *                 alias query); rows as in pa_cache_write_tokens.
 *   context_lens  lengths with the new tokens included; the n_s new queries
 *                 of sequence s sit at positions L_s - n_s .. L_s - 1 and
 *                 query i attends to keys 0 .. L_s - n_s + i.
 *   max_new_tokens  an upper bound on every n_s (sizes the launch grid); a
 *                 sequence with n_s > max_new_tokens produces no output rows.
 *   The pool must already hold the new tokens (pa_cache_write_tokens first,
 *   on the same stream).
 * No workspace.  Supported combinations, scales and errors as in pa_decode;
 * in addition PA_ERR_BAD_SHAPE when one pool block (2 * block_size *
 * num_kv_heads * head_dim elements) exceeds 4 GiB.  Any finite scale is
 * accepted, negative and zero included.
 * Sequences with n_s = 0, or with n_s > L_s, produce no output rows.
 */
pa_status pa_prefill(void* out, const void* query, pa_dtype q_dtype, const void* kv_pool, pa_dtype kv_dtype,
                     const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_seqlens,
                     int32_t num_seqs, int32_t num_tokens, int32_t max_new_tokens, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                     int32_t num_blocks, float scale, float k_scale, float v_scale, void* stream);

/*
 * pa_prefill_write -- pa_cache_write_tokens and pa_prefill in one call: the
 * prompt kernel writes the new tokens' K and V as it goes ([CANN notes
 * §4.2]).  With 16-bit KV this is one launch: each workgroup stores the rows
 * of the new tokens its own queries belong to, and the attention reads new
 * tokens from key / value rather than from the pool, so no workgroup waits
 * for another.  With fp8 KV (the attention must see the encoded codes) it is
 * the two launches, on the same stream.
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim] of src_dtype, rows as
 *                 in pa_cache_write_tokens; 16-bit KV needs src_dtype ==
 *                 kv_dtype (else PA_ERR_UNSUPPORTED); 16-byte aligned.
 *   The other arguments, the results and the errors are those of pa_prefill.
 *   The 16-bit form writes exactly the rows pa_prefill attends with (a
 *   sequence with n_s > L_s, or beyond max_new_tokens, is neither written nor
 *   attended); the pool afterwards is bit for bit what pa_cache_write_tokens
 *   leaves for every other sequence, and out is bit for bit pa_prefill's.
 */
pa_status pa_prefill_write(void* out, const void* query, pa_dtype q_dtype, void* kv_pool, pa_dtype kv_dtype,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* cu_seqlens,
                           int32_t num_seqs, int32_t num_tokens, int32_t max_new_tokens, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t num_blocks, float scale, float k_scale,
                           float v_scale, void* stream, const void* key, const void* value,
                           pa_dtype src_dtype);

/*
 * pa_copy_blocks -- copy whole KV blocks from one pool to another of the same
 * block geometry: for each pair i, block block_mapping[2i + 1] of dst_pool
 * becomes a byte copy of block block_mapping[2i] of src_pool (K half and V
 * half, every head: 2 * block_size * num_kv_heads * head_dim elements of
 * kv_dtype).  It serves the copy-on-write of a shared block before a branch
 * writes into it ([nano-vllm blog §4.3]; src_pool == dst_pool) and the swap
 * of a preempted request's blocks out to CPU memory and back in
 * ([nano-vllm blog §2.2]; one pool in pinned host memory).
 *
 *   src_pool, dst_pool  [src_num_blocks | dst_num_blocks, 2, block_size,
 *                       num_kv_heads, head_dim]; each is device memory of the
 *                       current device or host memory allocated pinned
 *                       (hipHostMalloc); anything else -> PA_ERR_UNSUPPORTED.
 *   block_mapping       device int32 [num_pairs, 2]: (source, destination).
 *                       No destination may appear twice, and within one pool
 *                       no block may be both a source and a destination
 *                       (pairs run in parallel).  Pairs with an id outside
 *                       its pool are skipped.
 *
 * Asynchronous on `stream`; num_pairs == 0 enqueues nothing.  Errors:
 * NULL_POINTER, MISALIGNED (pools and mapping need 16-byte alignment),
 * BAD_SHAPE (non-positive sizes, negative num_pairs), BAD_DTYPE,
 * UNSUPPORTED, HIP (launch failure).
 */
pa_status pa_copy_blocks(const void* src_pool, int32_t src_num_blocks, void* dst_pool,
                         int32_t dst_num_blocks, pa_dtype kv_dtype, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, const int32_t* block_mapping,
                         int32_t num_pairs, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The split-K workspace is a fixed array inside the
 * library, one copy per GPU, held until the process ends; the call itself
 * allocates nothing (no hipMalloc, no allocating library routine).
 *
 *   Arguments, results and errors are those of pa_decode without the
 *   workspace; partition_size 0 or a positive multiple of block_size.
 *   PA_ERR_WORKSPACE_TOO_SMALL when the call needs more workspace than the
 *   array holds: pa_decode_workspace_size(...) > pa_decode_noalloc_max_workspace()
 *   (64 MiB).  PA_ERR_HIP if the array's device address cannot be found.
 *
 * Every call on one GPU uses that GPU's one array, whose contents the last
 * call left (no call needs them cleared): calls that may overlap on one GPU
 * -- on different streams, or from different threads -- race on it and
 * must be ordered by the caller.
 */
pa_status pa_decode_noalloc(void* out, const void* query, pa_dtype q_dtype,
                            const void* kv_pool, pa_dtype kv_dtype,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                            float scale, float k_scale, float v_scale, int32_t partition_size,
                            void* stream);

/* Bytes of the fixed workspace pa_decode_noalloc uses on each GPU. */
size_t pa_decode_noalloc_max_workspace(void);

/* Human-readable name of a status value (static storage, never NULL). */
const char* pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
