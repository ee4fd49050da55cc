/*
 * pa_block_manager.h -- host-side KV block manager of libpagedkv.
 *
 * The step upstream of the device calls in pa.h: it decides which physical
 * block every token of every sequence lives in and emits the three arrays the
 * device path consumes -- block tables and context lengths for
 * pa_decode_attention, slot ids for pa_kv_append, (src, dst) pairs for
 * pa_block_copy.
 *
 * What the pages define (vLLM/PagedAttention paged-KV analysis page, sections
 * 2.2, 2.3, 3.2, 3.3 and 4.2; vLLM entity page, "what it is"):
 *   - one global allocator owns the physical blocks of the pool;
 *   - each sequence has its own block table from logical to physical blocks;
 *   - a sequence takes a new block only when its last one is full;
 *   - parallel samples, beams and common prompts share blocks by reference
 *     count, and a sequence about to write into a block that others still
 *     reference first gets a private copy (copy-on-write);
 *   - a finished sequence returns its blocks at once;
 *   - utilisation = sum of sequence lengths / (blocks in use * block size).
 * Where the pages are silent this library reads them as follows:
 *   - the lowest-numbered free block is taken first;
 *   - a fork starts with its parent's length and table, and every block of
 *     that table gains a reference;
 *   - a batch of appends is all-or-nothing (on PA_ERR_NO_BLOCKS nothing
 *     changes, so the caller can preempt and retry);
 *   - the copies a batch emits must be applied (pa_block_copy) before the
 *     tokens are written (pa_kv_append), both on one stream;
 *   - preemption evicts all of a request's blocks at once (Cross-Paper
 *     Synthesis page, section 3): a swapped-out sequence keeps its length
 *     but holds no block; on swap-in it gets fresh blocks (blocks it shared
 *     before come back as private copies).
 *
 * Every pointer here is HOST memory owned by the caller; no call touches the
 * GPU.  A manager is not thread-safe: calls on one manager must not overlap.
 * Separate managers are independent.
 */
#ifndef PAGEDKV_PA_BLOCK_MANAGER_H
#define PAGEDKV_PA_BLOCK_MANAGER_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* New manager of blocks 0 .. num_blocks-1 of block_size tokens each, all
 * free.  num_blocks in [1, 2^31 - 1], block_size >= 1.  *out receives the
 * handle (PA_ERR_SHAPE on bad sizes, PA_ERR_NULL if out is NULL). */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out);

/* Release the manager and everything it holds.  NULL is a no-op. */
void pa_bm_destroy(pa_block_manager* bm);

/* New empty sequence; *seq_id receives its id.  Ids are 0, 1, 2, ... in the
 * order sequences are created (by add or fork) and are never reused. */
pa_status pa_bm_add_sequence(pa_block_manager* bm, int64_t* seq_id);

/* New sequence sharing every block of `parent` (parallel sampling, beam
 * search): same length, same table, one more reference on each block.
 * PA_ERR_SEQUENCE if parent is not a live sequence. */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t* child);

/* Drop the sequence: every block of its table loses a reference, and blocks
 * left with none become free (a swapped-out sequence holds none).
 * PA_ERR_SEQUENCE if it is neither resident nor swapped out. */
pa_status pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);

/* Reserve num_new[i] token positions at the end of sequence seq_ids[i], for
 * i = 0 .. num_seqs-1 in order (a sequence may appear more than once).  For a
 * new position p of a sequence:
 *   p % block_size == 0          -> a fresh block is appended to its table;
 *   else, last block shared      -> copy-on-write: a fresh block replaces it
 *                                   in this table and (old, fresh) is emitted;
 *   slot = table[p / block_size] * block_size + p % block_size.
 *   slot_mapping   HOST int64 [slot_capacity]; receives sum(num_new) slots in
 *                  batch order
 *   block_mapping  HOST int32 [pair_capacity][2]; receives the (src, dst)
 *                  copies; at most one per entry of seq_ids
 *   num_pairs      HOST; receives the number of pairs written
 * Errors, all leaving the manager unchanged: PA_ERR_NULL, PA_ERR_SHAPE
 * (num_seqs < 0 or a negative count), PA_ERR_SEQUENCE (an id not live),
 * PA_ERR_CAPACITY (slot_capacity < sum(num_new) or pair_capacity too small
 * for the copies), PA_ERR_NO_BLOCKS (the free blocks do not cover the batch). */
pa_status pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* num_new,
                             int32_t num_seqs, int64_t* slot_mapping, int64_t slot_capacity,
                             int32_t* block_mapping, int32_t pair_capacity, int32_t* num_pairs);

/* Block tables and lengths of a batch of sequences, in the layout
 * pa_decode_attention reads: block_tables HOST int32
 * [num_seqs][max_blocks_per_seq] (entries past a sequence's last block are
 * -1), context_lens HOST int32 [num_seqs].  PA_ERR_SEQUENCE for an id not
 * live, PA_ERR_CAPACITY if a table is longer than max_blocks_per_seq or a
 * length exceeds INT32_MAX. */
pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                             int32_t max_blocks_per_seq, int32_t* block_tables,
                             int32_t* context_lens);

/* Prompt in large pages (Cross-Paper Synthesis page, section 5, the adaptive
 * block size item: huge pages where a prompt is written in one go).  Sequence
 * seq_id must be resident and empty (else PA_ERR_SHAPE).  Its first
 * floor(num_tokens / (pages_per_large * block_size)) large pages' worth of
 * tokens go to large pages -- each the lowest aligned run of pages_per_large
 * free blocks [P H, P H + H) -- and the remaining tokens to small blocks as
 * pa_bm_append_slots would place them.  slot_mapping (HOST int64
 * [slot_capacity]) receives num_tokens slots in token order.  pages_per_large
 * is a power of two in [1, 1024].  All-or-nothing: PA_ERR_NO_BLOCKS (no free
 * aligned run, or too few blocks) or PA_ERR_CAPACITY leave it empty.  Large
 * pages are always full, so no later append copies one; they are shared by
 * forks and returned block by block on free; a swap-in brings the sequence
 * back in small blocks. */
pa_status pa_bm_append_prompt_large(pa_block_manager* bm, int64_t seq_id, int32_t num_tokens,
                                    int32_t pages_per_large, int64_t* slot_mapping, int64_t slot_capacity);

/* Two-level tables of a batch, in the layout pa_decode_attention_hier reads:
 * large_tables HOST int32 [num_seqs][max_large_per_seq] (large-page ids,
 * -1 past the last), num_large HOST int32 [num_seqs], small_tables HOST int32
 * [num_seqs][max_small_per_seq] (-1 past the last), context_lens HOST int32
 * [num_seqs].  A sequence without large pages of this pages_per_large reports
 * num_large = 0 and all its blocks as small ones.  PA_ERR_SEQUENCE for an id
 * not resident, PA_ERR_CAPACITY if a row does not fit. */
pa_status pa_bm_block_tables_hier(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                                  int32_t pages_per_large, int32_t max_large_per_seq, int32_t max_small_per_seq,
                                  int32_t* large_tables, int32_t* num_large, int32_t* small_tables,
                                  int32_t* context_lens);

/* Preemption, out: the blocks of resident sequence seq_id in table order go
 * to block_ids (HOST int32 [capacity]; *num_ids receives the count), each
 * loses the sequence's reference (blocks left with none become free), and
 * the sequence becomes swapped out.  The caller copies the listed blocks to
 * host memory (pa_swap_out) before any work that may write them.  A swapped
 * sequence may only be named by pa_bm_swap_in, pa_bm_free_sequence and
 * pa_bm_sequence_length; elsewhere it is PA_ERR_SEQUENCE.  PA_ERR_CAPACITY
 * (nothing changes) if its table is longer than capacity. */
pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq_id, int32_t* block_ids, int32_t capacity,
                         int32_t* num_ids);

/* Preemption, back: a swapped-out sequence takes as many fresh blocks as it
 * held (lowest first), in table order, into block_ids (HOST int32
 * [capacity]); the caller copies the host data into them (pa_swap_in).
 * All-or-nothing: PA_ERR_NO_BLOCKS or PA_ERR_CAPACITY leave it swapped out. */
pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq_id, int32_t* block_ids, int32_t capacity,
                        int32_t* num_ids);

/* Number of free blocks (-1 if bm is NULL). */
int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/* Length in tokens of a sequence, resident or swapped out. */
pa_status pa_bm_sequence_length(const pa_block_manager* bm, int64_t seq_id, int64_t* length);

/* Utilisation as an exact ratio: *tokens = sum of the lengths of the
 * resident sequences, *slots = blocks in use * block_size (paged-KV analysis page,
 * section 4.2).  A block shared by k sequences counts once in *slots and its
 * tokens k times in *tokens. */
pa_status pa_bm_utilisation(const pa_block_manager* bm, int64_t* tokens, int64_t* slots);

/* Reference count of every block: refcounts HOST int32 [count], count must
 * equal the manager's num_blocks (PA_ERR_SHAPE otherwise).  For inspection
 * and tests. */
pa_status pa_bm_refcounts(const pa_block_manager* bm, int32_t* refcounts, int32_t count);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PA_BLOCK_MANAGER_H */
