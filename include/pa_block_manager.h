/*
 * pa_block_manager.h -- the host-side block manager around the paged-KV
 * kernels of pa.h: which physical block of the pool each sequence's logical
 * block is, which slot each new token goes to, and which blocks must be
 * copied before a shared block is written.
 *
 * The behaviour is the one the PagedAttention pages describe:
 *   - "What problem does PagedAttention solve, and what is continuous
 *     batching?" (datarekha), section "How PagedAttention works": the KV
 *     cache is a pool of fixed-size blocks; a per-request block table maps
 *     logical block to physical block; the allocator can take any free
 *     block; the last, partly filled block wastes at most the rest of one
 *     block; candidates with an identical prefix reference the same blocks,
 *     and when one diverges copy-on-write gives it a private block; prefix
 *     caching uses the same idea;
 *   - same page, "A concrete memory example": when a request finishes, its
 *     blocks return to the pool immediately;
 *   - same page, "A failure mode you can diagnose": the free KV-block count
 *     decides whether another request fits, not free device memory;
 *   - "Continuous Batching & Paged Attention" (topicspectrum), section
 *     "Paged attention borrows a trick from operating systems": a growing
 *     request attaches another block;
 *   - "PagedAttention & Continuous Batching" (ai-ml-animation-academy),
 *     section "If you remember three things": shared prefixes are shared
 *     blocks, which is prefix caching.
 *
 * The pages fix no allocation order; this manager fixes one:
 *   - free blocks form a FIFO queue, initially in the order given at
 *     creation (0..num_blocks-1 if none); a freed block joins the back;
 *   - a block that fills up is registered in the prefix cache under its
 *     content: the token ids it holds and the content of the blocks before
 *     it.  A registered block whose last user is freed stays cached, on a
 *     least-recently-freed list; allocation takes the queue first, then
 *     evicts the least recently freed cached block;
 *   - a sequence created from a prompt reuses the cached block of every
 *     full prompt block found in the cache, stopping at the first miss;
 *   - appending to a block that another sequence also references first gives
 *     the appending sequence a private copy, reported as a (src, dst) pair
 *     for pa_copy_blocks.
 *
 * Everything here runs on the host and touches no device memory: the caller
 * passes the slots to pa_reshape_and_cache, the pairs to pa_copy_blocks and
 * the tables to pa_decode.  A manager is safe to use from several threads
 * (calls are serialised internally).  An operation that cannot get the
 * blocks it needs returns PA_ERR_NO_BLOCKS and changes nothing; what to do
 * then (queue, preempt, reject) is the scheduler's choice.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;

/*
 * Creates a manager of num_blocks blocks of block_size token slots.
 * free_order (may be NULL: 0, 1, ...) is a permutation of 0..num_blocks-1,
 * the initial order of the free queue.  *out receives the handle.
 * Errors: PA_ERR_NULL (out), PA_ERR_SHAPE (sizes, or free_order not a
 * permutation).
 */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_bm** out);

/* Frees a manager (NULL is ignored). */
void pa_bm_destroy(pa_bm* bm);

/* Blocks an allocation could get now: the free queue plus cached blocks
 * nobody uses.  -1 for NULL. */
int32_t pa_bm_num_free(const pa_bm* bm);

/*
 * Starts sequence seq_id with num_tokens prompt tokens (token ids, used only
 * to recognise cached prefixes).  The longest run of leading full blocks
 * found in the prefix cache is reused; every other token gets a slot.
 * slots[i] (num_tokens entries) is the flat slot (block * block_size +
 * offset) where token i's keys and values go, or -1 for a token whose block
 * came from the cache (its keys and values are already there).
 * *num_cached receives the number of such leading tokens (a multiple of
 * block_size).  Errors: PA_ERR_NULL, PA_ERR_SHAPE (seq_id in use, negative
 * count), PA_ERR_NO_BLOCKS.
 */
pa_status pa_bm_add_sequence(pa_bm* bm, int64_t seq_id, const int32_t* tokens,
                             int32_t num_tokens, int32_t* slots, int32_t* num_cached);

/*
 * Appends num_tokens tokens to seq_id.  slots[i] receives token i's slot.
 * Copy-on-write: if the block receiving the first token is shared, the
 * sequence first gets a private block; cow_pairs (2 * cow_capacity int32,
 * may be NULL when cow_capacity is 0) receives the (src, dst) pairs to pass
 * to pa_copy_blocks before the append, *num_cow their number (0 or 1).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (unknown seq_id, negative count,
 * cow_capacity too small for the pair needed), PA_ERR_NO_BLOCKS.
 */
pa_status pa_bm_append(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                       int32_t* slots, int32_t* cow_pairs, int32_t cow_capacity,
                       int32_t* num_cow);

/*
 * One decode step's appends in one call: token tokens[i] is appended to
 * sequence seq_ids[i] for i in order, exactly as num_seqs single-token
 * pa_bm_append calls would do it, and slots[i] receives its slot.  The copy
 * pairs of all of them go to cow_pairs (2 * cow_capacity int32; num_seqs
 * pairs always suffice), *num_cow their number.  All or nothing: if the
 * pool cannot supply every block the whole step needs, nothing changes.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (unknown or repeated seq_id, negative
 * count, cow_capacity too small), PA_ERR_NO_BLOCKS.
 */
pa_status pa_bm_append_batch(pa_bm* bm, const int64_t* seq_ids, const int32_t* tokens,
                             int32_t num_seqs, int32_t* slots, int32_t* cow_pairs,
                             int32_t cow_capacity, int32_t* num_cow);

/*
 * Starts sequence child_id as a copy of parent_id that references the same
 * blocks (beam-search candidates): no block is copied until one of them
 * writes a shared block.  Errors: PA_ERR_SHAPE (unknown parent, child in
 * use).
 */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id);

/* Ends seq_id; blocks no other sequence references return to the pool.
 * Errors: PA_ERR_SHAPE (unknown seq_id). */
pa_status pa_bm_free(pa_bm* bm, int64_t seq_id);

/*
 * Block tables and lengths of num_seqs sequences, as pa_decode takes them:
 * tables[s * max_blocks_per_seq + j] = physical block of logical block j of
 * seq_ids[s], entries past the sequence's blocks set to pad_block;
 * seq_lens[s] = its token count.  Errors: PA_ERR_NULL, PA_ERR_SHAPE (unknown
 * id, or a sequence with more than max_blocks_per_seq blocks).
 */
pa_status pa_bm_tables(pa_bm* bm, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t pad_block, int32_t* tables,
                       int32_t* seq_lens);

/* Number of sequences that reference block `block` (0: free or only cached);
 * -1 for a bad handle or id. */
int32_t pa_bm_block_refs(const pa_bm* bm, int32_t block);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
