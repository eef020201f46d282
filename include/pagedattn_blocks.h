/*
 * libpagedattn block manager -- the host side of a paged KV cache: the pool of
 * physical blocks, each sequence's block table, reference-counted sharing of
 * blocks between forked sequences with copy-on-write, and the per-step index
 * arrays the device calls in pagedattn.h consume (slot_mapping for
 * kv_cache_write, src/dst pairs for copy_blocks, block_tables and
 * context_lens for paged_attention_decode).
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "vLLM 深度拆解：当大模型推理学会「分页注意力」..." (chenxutan.com/d/4834.html),
 *       section 2.1 (fixed-size blocks, block table, blocks returned to the
 *       free pool when a request ends) and section 3.3 (BlockSpaceManager:
 *       append_slot writes into the current block until it is full, then takes
 *       a new one; free returns every block; shared blocks are copied on write).
 *  [P3] the vLLM PagedAttention walkthrough at
 *       devpress.csdn.net/amd/6a31086710ee7a33f27dd05a.html, sections
 *       "关键设计一：分页管理" (a global pool whose free list starts as 0..N-1
 *       and hands out the last free block; out of memory when it is empty) and
 *       "关键设计二：Copy-on-Write" (a forked child shares the parent's blocks;
 *       appending to a shared last block first copies it to a new block and
 *       drops one reference to the old one).
 *
 * Readings where the pages are loose: blocks are reference counted, and a
 * block returns to the free list when its count reaches zero (the page's
 * code frees the old block outright, although its own comment speaks of
 * lowering a reference count); the slot of position t is table[t / B] * B +
 * t % B; a
 * new block is needed exactly when the new position is a multiple of B.
 *
 * The manager is host memory only and not thread safe: calls on one manager
 * must not overlap.  Sequence ids are caller-chosen int64 values.  Every call
 * returns a pa_status (pagedattn.h) or a count; nothing aborts or throws.
 */
#ifndef PAGEDATTN_BLOCKS_H
#define PAGEDATTN_BLOCKS_H

#include <stdint.h>

#include "pagedattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

typedef struct pa_block_stats {
  int32_t num_blocks;       /* pool size */
  int32_t free_blocks;      /* blocks on the free list */
  int32_t shared_blocks;    /* blocks referenced by more than one sequence */
  int32_t num_sequences;
  int64_t tokens_logical;   /* sum of the sequences' lengths */
  int64_t tokens_stored;    /* filled slots of used blocks, a shared slot once */
  int64_t slots_allocated;  /* used blocks * block_size */
  double utilisation;       /* tokens_stored / slots_allocated (1 when empty) */
} pa_block_stats;

/* A manager over num_blocks blocks of block_size tokens (block_size a power
 * of two in [1, 1024]); NULL on bad sizes or allocation failure. */
pa_block_manager *pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager *bm);

/* Free blocks now; whether a new sequence of num_tokens tokens fits (1 or 0). */
int32_t pa_bm_num_free_blocks(const pa_block_manager *bm);
int32_t pa_bm_can_allocate(const pa_block_manager *bm, int32_t num_tokens);

/* Admits a sequence whose first num_tokens tokens (its prompt, >= 0) are to be
 * stored: takes ceil(num_tokens / block_size) blocks.  slots (host, may be
 * NULL) receives the slot of every position 0 .. num_tokens-1, ready for
 * kv_cache_write.  Errors: PA_ERR_SEQ_EXISTS, PA_ERR_OOM (nothing taken),
 * PA_ERR_SHAPE. */
int32_t pa_bm_add_sequence(pa_block_manager *bm, int64_t seq_id, int32_t num_tokens,
                           int32_t *slots);

/* child starts as a copy of parent's block table (every block gains a
 * reference) and length.  Errors: PA_ERR_NO_SEQ, PA_ERR_SEQ_EXISTS. */
int32_t pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child);

/* Reserves the slot of the sequence's next position and grows its length by
 * one.  When that position opens a block, a block is taken; when it falls in
 * the last block and that block is shared, the block is first copied into a
 * new one: *copy_src / *copy_dst receive the pair for copy_blocks (both -1
 * when there is none).  Errors: PA_ERR_NO_SEQ, PA_ERR_OOM (state unchanged). */
int32_t pa_bm_append_slot(pa_block_manager *bm, int64_t seq_id, int32_t *slot,
                          int32_t *copy_src, int32_t *copy_dst);

/* Drops the sequence: every block loses a reference and returns to the free
 * list at zero.  Errors: PA_ERR_NO_SEQ. */
int32_t pa_bm_free_sequence(pa_block_manager *bm, int64_t seq_id);

/* The sequence's length (>= 0) or PA_ERR_NO_SEQ. */
int32_t pa_bm_context_len(const pa_block_manager *bm, int64_t seq_id);

/* Copies the sequence's block table into table[0 .. capacity) and returns its
 * number of blocks (which may exceed capacity: only capacity are written), or
 * PA_ERR_NO_SEQ. */
int32_t pa_bm_block_table(const pa_block_manager *bm, int64_t seq_id, int32_t *table,
                          int32_t capacity);

/* One decode step for n sequences: appends one slot to each, in order (see
 * pa_bm_append_slot), then writes the device inputs of the step into host
 * arrays:
 *   slot_mapping  [n]                  the new tokens' slots
 *   copy_pairs    [n][2]               copy-on-write pairs, *num_pairs of them
 *   block_tables  [n][max_blocks]      tables after the appends, unused
 *                                      entries set to pad_block
 *   context_lens  [n]                  lengths after the appends
 * Fails without changing anything (PA_ERR_OOM) when the free blocks cannot
 * cover the step; PA_ERR_SHAPE when a table would not fit max_blocks;
 * PA_ERR_NO_SEQ / PA_ERR_SEQ_EXISTS for unknown or repeated ids. */
int32_t pa_bm_prepare_decode(pa_block_manager *bm, const int64_t *seq_ids, int32_t n,
                             int32_t max_blocks, int32_t pad_block, int32_t *slot_mapping,
                             int32_t *copy_pairs, int32_t *num_pairs, int32_t *block_tables,
                             int32_t *context_lens);

/* Pool occupancy and utilisation. */
int32_t pa_bm_stats(const pa_block_manager *bm, pa_block_stats *out);

/*
 * pa_prefix_groups -- the shared-prefix groups of a decode batch, for
 * paged_attention_decode_prefix, found from the host copy of its block tables
 * ([P1] section 5.2 prefix caching and [P3] "关键设计二": sequences that share
 * a prompt prefix or were forked hold the same physical blocks at the same
 * logical positions).
 *
 * Scans the sequences in order; a group is a run of at least two
 * consecutive non-empty sequences, at most max_members long, whose rows start
 * with the same block.  Its reference row is the member with the most blocks
 * (the first of equals); every other member's shared length is
 * min(L, B * (leading entries equal to the reference row's, among the used
 * entries of both)), or 0 below min_shared_tokens, and the reference member's
 * is min(L, the longest of the others').  Every member thus names the
 * reference row's blocks below its shared length, and so every pair of
 * members names the same blocks below the shorter of its two.  A run in
 * which nobody shares min_shared_tokens is no group.  Sequences in no group
 * get shared length 0.
 *
 *   block_tables   host int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   host int32 [num_seqs]
 *   max_members    most members per group: 64 / G for the decode kernel
 *   groups         host int32 [num_seqs][2] out: (first sequence, members)
 *                  per group, ascending
 *   shared_lens    host int32 [num_seqs] out
 * Returns the number of groups (>= 0), or PA_ERR_NULL / PA_ERR_SHAPE.
 */
int32_t pa_prefix_groups(const int32_t *block_tables, const int32_t *context_lens,
                         int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                         int32_t max_members, int32_t min_shared_tokens, int32_t *groups,
                         int32_t *shared_lens);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_BLOCKS_H */
