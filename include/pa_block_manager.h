/*
 * pa_block_manager.h -- host-side manager of the paged KV pool with a prefix
 * cache.  Part of libpa.so; host code only (no GPU calls).
 *
 * What it keeps, after the pages:
 *   - a pool of num_blocks physical blocks of block_size tokens, handed out
 *     from a free queue; "KV cache block pool exhausted" is
 *     PA_ERR_POOL_EXHAUSTED ([nano-vllm blog §2.2]);
 *   - one block table per sequence (logical block -> physical block,
 *     [nano-vllm blog §2.2], [CANN notes §2.2]); a new block is taken only
 *     when the tail block is full ([nano-vllm blog §2.2], [CANN notes §2.3]);
 *   - reference counts: a block may sit in several tables ([vLLM notes,
 *     引用计数与 LRU]); a block is writable only while one table holds it;
 *   - a prefix cache over FULL blocks only ([vLLM notes, 边界条件]: 100
 *     tokens -> at most 96 cached).  Each full block gets a chained hash
 *     H(hash of the previous block, the block's token ids, extra key), the
 *     first block chaining from a fixed initial value ([vLLM notes, 链式哈希];
 *     the extra key separates model versions, adapters, salts --
 *     [nano-vllm blog §3.2]).  A new sequence walks its prompt block by block
 *     and reuses every cached block up to the first miss ([vLLM notes, 查找与
 *     复用], [nano-vllm blog §3.2], [nano-vllm blog §4.3]).  A hit is also
 *     checked token for token against the cached block's own tokens and
 *     predecessor, so a hash collision is never reused ([nano-vllm blog §3.2]
 *     advises checking).
 *   - blocks whose count drops to 0 keep their cache entry and go to the
 *     most-recently-used end of the free queue; allocation takes the least
 *     recently used block and drops its cache entry ([vLLM notes, 引用计数与
 *     LRU]).  A sequence's blocks are released tail first, so its prefix
 *     blocks -- the ones most likely to be shared -- are evicted last.
 *   - fork (parallel sampling, beam search) shares every block of the parent;
 *     appending into a shared tail block first moves the child to a fresh
 *     copy (copy-on-write, [nano-vllm blog §4.3]); the (source, destination)
 *     pairs to copy are queued for the caller to run with pa_copy_blocks.
 *
 * Hash: 64-bit FNV-1a over the little-endian bytes of (previous hash, token
 * ids, extra key).  Not thread-safe: one manager per scheduler thread, or a
 * lock around every call.  Every call either succeeds completely or leaves
 * the manager unchanged.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;    /* opaque */

typedef struct pa_bm_stats {
    int32_t num_blocks;        /* pool size                                          */
    int32_t free_blocks;       /* blocks in the free queue (reference count 0)       */
    int32_t cached_free_blocks;/* of those, blocks still holding a cache entry        */
    int32_t cached_blocks;     /* cache entries (full blocks findable by hash)        */
    int32_t num_sequences;
    int64_t lookups;           /* full prompt blocks looked up by pa_bm_add_sequence  */
    int64_t hits;              /* of those, blocks reused from the cache              */
    int64_t evictions;         /* cache entries dropped to allocate their block       */
} pa_bm_stats;

/* A manager of num_blocks blocks of block_size tokens (both > 0).
 * initial_order: NULL, or a permutation of 0..num_blocks-1 giving the free
 * queue's initial order (least recently used first).  Returns NULL on bad
 * arguments or allocation failure. */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, uint64_t extra_key,
                    const int32_t* initial_order);
void pa_bm_destroy(pa_bm* bm);

/* Admit sequence seq_id (not already present) with its prompt tokens
 * [num_tokens >= 0]: reuse cached full blocks from the start up to the first
 * miss, then allocate blocks for the rest.  *cached_tokens (may be NULL)
 * receives the number of prompt tokens whose KV is already in the reused
 * blocks (a multiple of block_size); the caller computes and writes only
 * tokens cached_tokens .. num_tokens-1.  The newly allocated full blocks
 * become findable at once: their KV must be written before another
 * sequence's attention reads them.  Errors: NULL_POINTER, BAD_SHAPE (bad
 * count or id already present), POOL_EXHAUSTED. */
pa_status pa_bm_add_sequence(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                             int32_t* cached_tokens);

/* Append one generated token: the token goes to the tail block if it has
 * room (copy-on-write first when that block is shared), otherwise to a new
 * block.  A block that becomes full enters the prefix cache.  Errors:
 * NULL_POINTER, UNKNOWN_SEQUENCE, POOL_EXHAUSTED. */
pa_status pa_bm_append_token(pa_bm* bm, int64_t seq_id, int32_t token);

/* New sequence child_id sharing every block (and the tokens) of parent_id.
 * Errors: NULL_POINTER, UNKNOWN_SEQUENCE, BAD_SHAPE (child id present). */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id);

/* Release a finished sequence: every block loses one reference, tail first;
 * blocks reaching 0 go to the free queue keeping their cache entries.
 * Errors: NULL_POINTER, UNKNOWN_SEQUENCE. */
pa_status pa_bm_free_sequence(pa_bm* bm, int64_t seq_id);

/* Move up to max_pairs queued copy-on-write copies, as (source block,
 * destination block) int32 pairs, into pairs[2 * max_pairs]; returns how many
 * were moved (oldest first), -1 for a NULL manager.  Run them with
 * pa_copy_blocks (src_pool == dst_pool) before the next attention. */
int32_t pa_bm_take_copies(pa_bm* bm, int32_t* pairs, int32_t max_pairs);

/* Tokens held by seq_id, or -1 when unknown. */
int32_t pa_bm_sequence_length(const pa_bm* bm, int64_t seq_id);

/* Copy seq_id's block table into out[0 .. max_blocks-1] (as far as it fits);
 * returns the table's length, or -1 when unknown. */
int32_t pa_bm_block_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t max_blocks);

/* Reference count of one physical block (-1 out of range). */
int32_t pa_bm_ref_count(const pa_bm* bm, int32_t block);

pa_status pa_bm_stats_get(const pa_bm* bm, pa_bm_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
