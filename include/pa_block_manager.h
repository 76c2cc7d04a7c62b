/*
 * pa_block_manager.h -- host-side block manager of the paged KV cache (C ABI, part of libpa.so).
 *
 * It decides which physical block of the pool holds each position of each sequence; the device
 * entry points of pa.h then take its output: new tokens' slots (pa_reshape_and_cache), block
 * tables (pa_decode, pa_prefill_chunk) and copy-on-write pairs (pa_copy_blocks). The rules are the
 * pages':
 *   [MEM] openeuler.csdn.net "高并发 AI 服务的内存瓶颈":
 *         "机制1：按需分配" -- a sequence of L tokens holds ceil(L/16) blocks; a new block is taken
 *         only when the last one is full (worked example: 100 tokens -> 7 blocks, 112 slots);
 *         "Block Table 数据结构" -- position i is stored at slot table[i / 16] * 16 + i % 16;
 *         "机制 2：写时复制" -- parallel samples share their prompt's blocks with a reference count
 *         and get a private block only where they diverge (worked example: 3 samples of a 5-block
 *         prompt hold 8 blocks instead of 18).
 *   [V1]  lilinji.mintlify.site lecture 34 "vLLM 生产级系统架构全景剖析…":
 *         §1.2 -- allocate_slots(req, num_tokens) appends into the last block while it has room and
 *         else takes a new block from the pool; free(req) releases a request's blocks in reverse
 *         order (tail first, prompt blocks last); the pool keeps its free blocks in a doubly linked
 *         queue so that a cached free block can be taken out of the middle in O(1);
 *         §2.2 -- a new request's longest run of leading blocks already in the prefix cache is
 *         shared (reference count + 1) instead of recomputed;
 *         §2.3 -- a block whose count falls to 0 keeps its contents and stays findable ("cached
 *         free") at the tail of the free queue; allocation takes blocks from the head, so the
 *         least recently freed cached block is evicted first, and a block in use is never evicted.
 *
 * Conventions
 * -----------
 *  - Every pointer argument is HOST memory owned by the caller. The manager allocates its own
 *    host memory (create .. destroy) and never touches device memory.
 *  - A manager is not thread-safe: calls on one manager must be serialised by the caller. Distinct
 *    managers are independent.
 *  - Sequence ids are caller-chosen int64 values, unique among live sequences.
 *  - A failed call returns its status, leaves the manager exactly as it was and sets the calling
 *    thread's pa_last_error() message. PA_ERR_INVALID_ARG: bad pointer, count, unknown or duplicate
 *    sequence id, or a token_ids/NULL mix a call does not allow. PA_ERR_NO_BLOCKS: the free queue
 *    holds fewer blocks than the call needs.
 *  - Prefix cache: only FULL blocks whose 16 token ids are all known are cached. A block is found
 *    by its content: the ids of every token from position 0 up to the block's end. The manager
 *    keys this by a 64-bit hash chained over blocks and, on a hit, compares the block's own 16 ids
 *    and its parent's hash; a false hit needs a 64-bit collision of two different parent chains.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/*
 * pa_bm_create -- a manager of num_blocks (> 0) physical blocks, all free. free_order (may be
 * NULL = 0, 1, .., num_blocks-1) is a permutation of the block ids giving the initial free queue
 * from head to tail. prefix_caching != 0 turns the prefix cache on. *out receives the handle.
 */
pa_status_t pa_bm_create(int32_t num_blocks, const int32_t *free_order, int32_t prefix_caching,
                         pa_block_manager **out);

/* pa_bm_destroy -- release the manager (NULL is a no-op). Live sequences are dropped with it. */
void pa_bm_destroy(pa_block_manager *bm);

/* pa_bm_add_sequence -- a new sequence with no tokens and no blocks. */
pa_status_t pa_bm_add_sequence(pa_block_manager *bm, int64_t seq_id);

/*
 * pa_bm_match_prefix -- [V1] §2.2 longest prefix match for a new, still empty sequence (prefix
 * caching on). token_ids [num_tokens] is its prompt. The longest run of leading full blocks whose
 * contents are in the cache is shared, at most (num_tokens - 1) / 16 blocks so that at least the
 * last prompt token is left to compute. Each shared block's reference count rises by one; a cached
 * free block (count 0) leaves the free queue. *num_cached_tokens = 16 * blocks shared; the
 * sequence then holds that many tokens. With prefix caching off it shares nothing (*num_cached
 * = 0). The caller appends the remaining prompt tokens with pa_bm_allocate_slots.
 */
pa_status_t pa_bm_match_prefix(pa_block_manager *bm, int64_t seq_id, const int32_t *token_ids,
                               int32_t num_tokens, int32_t *num_cached_tokens);

/*
 * pa_bm_allocate_slots -- [V1] §1.2 allocate_slots: append num_tokens (>= 0) positions to the
 * sequence and write their slots to slots[0 .. num_tokens-1] (position i -> table[i/16]*16 + i%16).
 * New blocks come from the head of the free queue; a cached free block taken there is evicted
 * from the prefix cache. If the first new position falls in a partly filled last block that other
 * sequences share (reference count > 1), that block is copied on write ([MEM] 机制 2): a new block
 * replaces it in this sequence's table, the shared block loses one reference, and cow_pair receives
 * (shared block, new block) for pa_copy_blocks, which must run before the new tokens are written;
 * otherwise cow_pair receives (-1, -1). At most one copy arises per call.
 * token_ids [num_tokens] (may be NULL) are the appended tokens' ids: with prefix caching on, every
 * block they complete is entered in the cache (unless a block with the same contents already is).
 * Once a sequence has appended tokens without ids, none of its later blocks is cached.
 */
pa_status_t pa_bm_allocate_slots(pa_block_manager *bm, int64_t seq_id, const int32_t *token_ids,
                                 int32_t num_tokens, int32_t *slots, int32_t cow_pair[2]);

/*
 * pa_bm_fork -- [MEM] 机制 2 parallel sampling / beam search: a new sequence child_id that shares
 * every block of parent_id (each block's reference count + 1) and holds the same tokens.
 */
pa_status_t pa_bm_fork(pa_block_manager *bm, int64_t parent_id, int64_t child_id);

/*
 * pa_bm_free -- [V1] §1.2 free(req): drop the sequence, releasing its blocks from the last to the
 * first. A block whose reference count falls to 0 goes to the tail of the free queue; a cached
 * block stays in the prefix cache until it is evicted.
 */
pa_status_t pa_bm_free(pa_block_manager *bm, int64_t seq_id);

/* Number of tokens the sequence holds and number of blocks in its table. */
pa_status_t pa_bm_sequence_info(const pa_block_manager *bm, int64_t seq_id, int32_t *num_tokens,
                                int32_t *num_blocks);

/*
 * pa_bm_block_tables -- block tables of num_seqs sequences as the rows of out
 * [num_seqs][max_blocks_per_seq] (the pa_decode / pa_prefill_chunk layout), padded with -1.
 * PA_ERR_INVALID_ARG if a sequence holds more than max_blocks_per_seq blocks.
 */
pa_status_t pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seq_ids,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t *out);

/* Blocks in the free queue (fresh or cached free): what allocation can still take. */
int32_t pa_bm_num_free_blocks(const pa_block_manager *bm);

/*
 * pa_bm_free_queue -- the free queue from head (next to be taken) to tail into out[0 .. n-1],
 * n = min(capacity, pa_bm_num_free_blocks); returns n (or -1 on a NULL argument).
 */
int32_t pa_bm_free_queue(const pa_block_manager *bm, int32_t *out, int32_t capacity);

/*
 * pa_bm_block_state -- reference count of block `block` and whether it is in the prefix cache
 * (is_cached may be NULL).
 */
pa_status_t pa_bm_block_state(const pa_block_manager *bm, int32_t block, int32_t *ref_cnt,
                              int32_t *is_cached);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
