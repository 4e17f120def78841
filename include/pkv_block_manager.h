/*
 * pkv_block_manager.h - host-side block manager for the paged KV cache.
 *
 * The bookkeeping the decode path needs before each step (supersilo.blog
 * vLLM/PagedAttention summary, sections "PagedAttention의 설계" and "블록
 * 공유"; blog.aqudi.me "벤치마크가 다가 아니야! vLLM으로 보는 LLM 추론
 * 최적화", section 3):
 *   - blocks are allocated on demand: a sequence gets a new block only when
 *     its last one is full, so at most the last block of a sequence has free
 *     slots;
 *   - several sequences may point at the same physical block (parallel
 *     sampling, beam search: a forked sequence shares all of its parent's
 *     blocks), counted by a per-block reference count;
 *   - a shared block is copied only when one holder must write into it
 *     (copy-on-write): appending to a sequence whose last block is partly
 *     filled and shared gives that sequence a private copy and records the
 *     (source, destination) pair for pkv_copy_blocks. The last remaining
 *     holder writes in place.
 *
 * Allocation policy (fixed, so results are reproducible): free blocks form a
 * stack; initially block 0 is on top, then 1, 2, ...; a freed block is pushed
 * on top; blocks of a freed sequence are pushed in logical order (so its last
 * block is reused first).
 *
 * Swapping (supersilo.blog summary, section "적용 범위와 관련 연구": when
 * device memory runs short, sequences move to CPU memory and return later).
 * A manager may own a second pool of host blocks, with its own free stack
 * (same policy) and reference counts. Swapping a set of sequences out gives
 * every distinct device block they hold one host block (a block shared
 * inside the set moves once and stays shared) and drops their device
 * references; swapping in is the mirror image. The returned pairs are what
 * pkv_swap_blocks (pkv_swap.h) must copy. Within one step, run the work in
 * this order on one stream: the swap-out copies, the swap-in copies, the
 * copy-on-write copies, then the append (a block freed by a swap-out may be
 * the target of a later copy). A swap is refused while copy-on-write pairs
 * are queued (take and run them first), since the swap's copies would read
 * blocks those pairs have not filled yet. A swapped-out sequence cannot be
 * appended to, forked or put in a batch until it is swapped in; it can be
 * freed.
 *
 * All functions are host-only and take plain host memory. A manager is not
 * thread-safe: calls on one manager must not overlap. Sequence ids are
 * arbitrary 64-bit integers chosen by the caller. Functions return a
 * pkv_status (negative on error, leaving the manager unchanged) unless
 * stated otherwise; PKV_ERR_NO_BLOCKS means an operation needed a free block
 * and the pool had none.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/* A manager for a pool of num_blocks blocks of block_size tokens (both > 0);
 * NULL on invalid sizes or allocation failure. */
PKV_API pkv_block_manager* pkv_bm_create(int num_blocks, int block_size);

/* The same with a host pool of num_host_blocks blocks (>= 0) to swap to. */
PKV_API pkv_block_manager* pkv_bm_create_swappable(int num_blocks, int num_host_blocks,
                                                   int block_size);
PKV_API void pkv_bm_destroy(pkv_block_manager* bm);

/* A new, empty sequence (PKV_ERR_INVALID if the id exists). */
PKV_API int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id);

/* child becomes a sequence with the parent's length and the parent's blocks,
 * each of whose reference counts goes up by one. */
PKV_API int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Reserve the slot of the sequence's next token and count the token:
 * *block / *offset receive the physical block and the slot inside it (what
 * pkv_kv_cache_append will write, given the table this leaves). Allocates a
 * block if the sequence is empty or its last block is full; copies the last
 * block on write if it is shared (the copy pair is queued, see
 * pkv_bm_take_copies). */
PKV_API int pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t* block,
                                int32_t* offset);

/* One decode step's worth of pkv_bm_append_token: the slots of the next
 * token of seq_ids[0..n) (distinct ids) in that order (the same result as n
 * single calls),
 * written to blocks[i] / offsets[i]. All or nothing: if the pool cannot
 * supply every block the step needs, PKV_ERR_NO_BLOCKS and no change. */
PKV_API int pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seq_ids, int n,
                                int32_t* blocks, int32_t* offsets);

/* Drop the sequence: every block's reference count goes down by one, and
 * blocks no longer referenced return to the free stack (the host stack for a
 * swapped-out sequence). PKV_ERR_INVALID, and no change, while
 * copy-on-write pairs are queued (take them first): a block released here
 * could otherwise be handed out again before those copies run, as a second
 * copy's destination or as a destination that is still a copy's source. */
PKV_API int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/* Swap the resident sequences seq_ids[0..n) (distinct) out to host blocks.
 * Writes the (device block, host block) pairs to copy, in order of first use
 * (the sequences in the given order, each table in logical order), to
 * pairs[2k], pairs[2k + 1]; returns their number. All or nothing:
 * PKV_ERR_NO_BLOCKS if the host pool has too few free blocks,
 * PKV_ERR_WORKSPACE if more than max_pairs pairs would be needed (num_blocks
 * always suffices), PKV_ERR_INVALID for an unknown, repeated or already
 * swapped id or while copy-on-write pairs are queued. */
PKV_API int pkv_bm_swap_out(pkv_block_manager* bm, const int64_t* seq_ids, int n,
                            int32_t* pairs, int max_pairs);

/* Swap the swapped-out sequences seq_ids[0..n) back in: (host block, device
 * block) pairs as for pkv_bm_swap_out (num_host_blocks always suffices);
 * PKV_ERR_NO_BLOCKS if the device pool has too few free blocks. */
PKV_API int pkv_bm_swap_in(pkv_block_manager* bm, const int64_t* seq_ids, int n,
                           int32_t* pairs, int max_pairs);

/* 1 if the sequence is swapped out, 0 if resident, PKV_ERR_INVALID if unknown. */
PKV_API int pkv_bm_is_swapped(const pkv_block_manager* bm, int64_t seq_id);

/* Free host blocks, or a negative status. */
PKV_API int pkv_bm_num_free_host_blocks(const pkv_block_manager* bm);

/* Reference count of a host block (0 = free), or PKV_ERR_INVALID. */
PKV_API int pkv_bm_host_refcount(const pkv_block_manager* bm, int32_t block);

/* Free blocks, or a negative status. */
PKV_API int pkv_bm_num_free_blocks(const pkv_block_manager* bm);

/* Length of a sequence in tokens, or PKV_ERR_INVALID for an unknown id. */
PKV_API int pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id);

/* Reference count of a physical block (0 = free), or PKV_ERR_INVALID. */
PKV_API int pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);

/* Copy the sequence's block table (logical -> physical; host blocks for a
 * swapped-out sequence) into out[0..); returns
 * the number of blocks, PKV_ERR_INVALID for an unknown id, or
 * PKV_ERR_WORKSPACE when max_blocks is too small. */
PKV_API int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* out,
                               int max_blocks);

/* Copy-on-write pairs queued since the last call, in the order they arose:
 * writes up to max_pairs (src, dst) pairs to pairs[2 * i], pairs[2 * i + 1]
 * and removes them from the queue; returns how many were written. */
PKV_API int pkv_bm_take_copies(pkv_block_manager* bm, int32_t* pairs, int max_pairs);

/* For pkv_paged_attention_decode_grouped: seq_ids[0..n) form groups of
 * group_size consecutive ids (n a multiple of group_size); shared_tokens[k]
 * receives block_size times the number of leading logical blocks that every
 * sequence of group k maps to the same physical block. Such a block has not
 * been written since it became shared (a write into a shared block copies
 * it first), so every sequence reads the same tokens from it.
 * PKV_ERR_INVALID for an unknown or swapped-out id. */
PKV_API int pkv_bm_shared_prefix(const pkv_block_manager* bm, const int64_t* seq_ids, int n,
                                 int group_size, int32_t* shared_tokens);

/* The launch inputs for a batch: row i of tables ([n][max_blocks], padded
 * with -1) and seq_lens[i] for seq_ids[i]. PKV_ERR_WORKSPACE if a sequence
 * has more than max_blocks blocks, PKV_ERR_INVALID if one is swapped out. */
PKV_API int pkv_bm_build_batch(const pkv_block_manager* bm, const int64_t* seq_ids, int n,
                               int32_t* tables, int max_blocks, int32_t* seq_lens);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
