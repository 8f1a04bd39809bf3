/*
 * pa_alloc.h -- host-side block allocator for the paged KV cache in pa.h.
 *
 * The cache is a pool of num_blocks physical blocks of block_size token
 * slots; each sequence owns a block table mapping its logical blocks to
 * physical ones; blocks are taken on demand as a sequence grows and go back
 * to the pool when it ends (tiniestgpt notes, "PagedAttention: why it is
 * needed"). With prefix caching on, every complete block is registered under
 * the chained hash h_i = H(h_{i-1}, token ids of block i), and a new
 * sequence whose leading complete blocks match registered ones shares those
 * blocks instead of computing them again (tiniestgpt notes, "Prefix
 * Caching": only complete blocks are cached).
 *
 * The allocator outputs exactly what the device entry points take: slot ids
 * (block * block_size + slot) for pa_cache_write, and a block table plus
 * sequence lengths for pa_decode / pa_verify. It runs on the host, allocates
 * host memory only, and touches no device memory.
 *
 * Rules where the notes leave a choice open:
 *   - H is 64-bit FNV-1a over the parent hash (8 bytes, little-endian) and
 *     then the block's token ids (4 bytes each, little-endian); the first
 *     block's parent is 0. Hits are taken on the 64-bit hash alone.
 *   - Matching is tried only while a sequence consists of prefix hits from
 *     its start, stops at the first miss, and never covers the block holding
 *     the call's last token (that token is computed, so the step has its
 *     logits). Cached positions get slot id -1, which pa_cache_write skips.
 *   - A block that fills is registered unless its hash is already taken.
 *   - Free blocks wait in one queue. A sequence's blocks are released last
 *     logical block first; a released block with a registration joins the
 *     back (it stays findable until reused), one without joins the front.
 *     A fresh block comes from the front and loses any old registration; a
 *     hit on a free block takes it out of the queue.
 *   - Every call succeeds whole or changes nothing (except
 *     pa_alloc_append_batch, see there).
 *
 * An allocator is not thread-safe: calls on one allocator must not overlap.
 * All pointers are host pointers owned by the caller. Errors return a
 * PA_ERR_* code from pa.h and leave a message for pa_last_error().
 */
#ifndef PA_ALLOC_H
#define PA_ALLOC_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_allocator pa_allocator; /* opaque */

/* Create an allocator over blocks 0 .. num_blocks-1 (all free, queued in
 * ascending order). block_size >= 1 (the kernels take 16). prefix_cache:
 * 0 off, 1 on. *out receives the allocator (NULL on failure).
 * PA_ERR_INVALID_ARG on bad sizes or a NULL out. */
int pa_alloc_create(int32_t num_blocks, int32_t block_size, int32_t prefix_cache, pa_allocator** out);

/* Free the allocator and everything it holds. NULL is a no-op. */
void pa_alloc_destroy(pa_allocator* a);

/* Start an empty sequence under the caller's id. PA_ERR_INVALID_ARG if the
 * id is live. */
int pa_alloc_add(pa_allocator* a, int64_t seq_id);

/* Start an empty ring sequence for a window layer (Lab 5, "Ring KV Cache"):
 * it takes blocks on demand until it holds ring_blocks >= 1 of them, after
 * which position t lives in slot t mod (ring_blocks * block_size) of its
 * blocks, overwriting the token ring_blocks * block_size positions earlier.
 * Its blocks are rewritten, so it never registers or matches a prefix. A
 * position that a later token of the same append overwrites gets slot id -1,
 * so pa_cache_write never writes one slot twice in a call. Its block table (ring_blocks entries once full) goes to the attention calls
 * with pa_args.ring_blocks = ring_blocks. PA_ERR_INVALID_ARG if the id is
 * live or ring_blocks < 1. */
int pa_alloc_add_ring(pa_allocator* a, int64_t seq_id, int32_t ring_blocks);

/* Grow sequence seq_id by n >= 0 tokens. tokens: NULL, or the n token ids
 * (needed for prefix caching; a sequence once grown without ids is never
 * registered or matched again). slot_ids: n outputs, the slot of each new
 * token, -1 where its keys and values are already cached. cached: NULL, or
 * receives how many leading tokens were prefix hits (a multiple of
 * block_size). PA_ERR_NO_BLOCKS if the pool cannot hold the growth
 * (nothing changes); PA_ERR_INVALID_ARG for an unknown id, n < 0, or a NULL
 * slot_ids with n > 0. */
int pa_alloc_append(pa_allocator* a, int64_t seq_id, int32_t n, const int32_t* tokens, int64_t* slot_ids,
                    int32_t* cached);

/* pa_alloc_append for num_seqs sequences in order (a batched decode or
 * prefill step): counts[i] tokens for seq_ids[i]; tokens (NULL, or all ids
 * concatenated in the same order) and slot_ids (outputs, concatenated) hold
 * sum(counts) entries; cached: NULL or num_seqs outputs. *done receives the
 * number of sequences fully appended. On an error the first *done sequences
 * keep their growth and the rest are untouched, so a scheduler can preempt
 * and retry from there. */
int pa_alloc_append_batch(pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids, const int32_t* counts,
                          const int32_t* tokens, int64_t* slot_ids, int32_t* cached, int32_t* done);

/* End sequence seq_id and return its blocks (shared blocks stay with their
 * other sequences). PA_ERR_INVALID_ARG for an unknown id. */
int pa_alloc_release(pa_allocator* a, int64_t seq_id);

/* Number of free blocks (queued, registered or not). -1 for a NULL allocator. */
int32_t pa_alloc_num_free(const pa_allocator* a);

/* Block table and lengths for num_seqs sequences: table is [num_seqs][max_blocks]
 * int32 (entries past a sequence's blocks are set to 0, never read by the
 * kernels), seq_lens [num_seqs] int32. PA_ERR_INVALID_ARG for an unknown id
 * or a sequence with more than max_blocks blocks or more than 2^31-1 tokens. */
int pa_alloc_block_table(const pa_allocator* a, int32_t num_seqs, const int64_t* seq_ids, int32_t max_blocks,
                         int32_t* table, int32_t* seq_lens);

/* Prefix-cache counters since creation: blocks looked up and blocks hit
 * (hit rate = hits / queried). Either pointer may be NULL. */
int pa_alloc_stats(const pa_allocator* a, int64_t* queried, int64_t* hits);

/* The free queue front to back, for inspection and tests: writes up to cap
 * block ids to out and the queue length to *count. */
int pa_alloc_free_queue(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* PA_ALLOC_H */
