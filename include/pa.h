/*
 * pa.h -- C ABI of the paged-attention hot path for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of PagedAttention as the pages state them:
 *   [MEM] openeuler.csdn.net "高并发 AI 服务的内存瓶颈": KV cache cut into fixed 16-token blocks
 *         reached through a per-sequence block table (sections "vLLM - PagedAttention",
 *         "Block Table 数据结构", "Attention 计算时的 Block 映射"); copy-on-write of shared blocks
 *         (section "机制 2：写时复制").
 *   [PD]  lilinji.mintlify.site lecture 32 "LLM 在线推理两阶段（Prefill vs Decode）…": attention
 *         softmax(Q K^T / sqrt(d_k)) V and the decode step that appends k_t, v_t and attends the whole
 *         history (§3.1); GQA head groups (§3.4); causal masking (§1.1); chunked prefill mixed with
 *         decodes under one token budget (§5.4, §5.5).
 *   [OV]  devpress.csdn.net/amd vLLM overview: per-block attention over the block table (§3 (3))
 *         combined with a running maximum and sum of exponentials (§9 (4) online softmax).
 *   [V1]  lilinji.mintlify.site lecture 34 "vLLM 生产级系统架构全景剖析…": §2.2 shared prefixes
 *         and block reference counts; §4.4 the FP8 (E4M3) KV cache, one byte per key and value
 *         element (kv_cache_dtype="fp8").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller, row-major and contiguous, and
 *    aligned to 16 bytes. These entry points allocate no memory, keep no state between calls (apart
 *    from a thread-local error message) and may be called from several threads. (The host-side
 *    block manager of pa_block_manager.h, also in this library, is the one stateful part;
 *    pa_decode_noalloc keeps its partial results in a static device array instead of a workspace.)
 *  - 16-bit element type: PA_DTYPE_F16 (IEEE binary16) or PA_DTYPE_BF16 (bfloat16). Queries, keys,
 *    values, caches and outputs all share it. Arithmetic is float32; outputs are rounded to nearest
 *    even.
 *  - FP8 caches ([V1] §4.4): the *_fp8 entry points keep k_cache and v_cache as E4M3 codes (the OCP
 *    8-bit format: sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, largest
 *    magnitude 448, S.1111.111 = NaN), one byte per element, same layout. Element = code value *
 *    k_scale (keys) or * v_scale (values), one finite positive scale per cache chosen by the caller.
 *    Their `dtype` argument is the 16-bit type of queries, new keys/values and outputs.
 *    pa_copy_blocks takes PA_DTYPE_FP8_E4M3 for such caches.
 *  - Cache layout: k_cache and v_cache are [num_blocks][num_kv_heads][PA_BLOCK_SIZE][head_dim].
 *    Slot s (the storage position of a token, physical_block * 16 + offset, [MEM] Block Table
 *    数据结构) is block s / 16, in-block offset s % 16; each (block, kv head) tile of 16 rows is
 *    contiguous.
 *  - scale (the softmax temperature, 1/sqrt(head_dim) for the pages' attention) must be finite and
 *    positive.
 *  - head_dim is 64 or 128. Query head h reads kv head h / (num_q_heads / num_kv_heads) ([PD] §3.4).
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue work: they return
 *    before it runs and never synchronise with the device.
 *  - Argument checks run on the host before anything is enqueued; a failed check returns its status
 *    and enqueues nothing. Index CONTENTS live on the device and are not read by the host. The
 *    kernels never access memory outside the arguments for any index values: a slot, block id or
 *    copy pair outside the pool is skipped (it writes nothing / contributes nothing), and a sequence
 *    length beyond the stated maximum is clamped to it. Such inputs give unspecified results, not
 *    faults.
 *  - Errors: PA_ERR_INVALID_ARG (bad pointer, alignment, count or size), PA_ERR_UNSUPPORTED (a
 *    head_dim or head-group size with no kernel), PA_ERR_WORKSPACE (workspace too small),
 *    PA_ERR_HIP (a launch failed), PA_ERR_NO_BLOCKS (block manager only). pa_last_error() gives
 *    the calling thread's last message.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,
    PA_ERR_UNSUPPORTED = 2,
    PA_ERR_WORKSPACE = 3,
    PA_ERR_HIP = 4,
    PA_ERR_NO_BLOCKS = 5 /* the block manager's free queue is too short (pa_block_manager.h) */
} pa_status_t;

typedef enum { PA_DTYPE_F16 = 0, PA_DTYPE_BF16 = 1, PA_DTYPE_FP8_E4M3 = 2 } pa_dtype_t;

/*
 * pa_reshape_and_cache -- write the new tokens' keys and values into their cache slots.
 * [PD] §3.1: a decode step computes k_t, v_t and appends them to the cache; [OV] §8 (1)(2): each
 * layer stores its new K and V into the paged cache; [MEM] Block Table 数据结构: the slot of a
 * position is physical_block * 16 + offset.
 *   key, value    [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping  [num_tokens] int32; token t goes to slot slot_mapping[t]; a negative slot means
 *                 "skip this token". Slots in one call must be distinct (else the surviving write is
 *                 unspecified). The values are copied bit for bit.
 *   k_cache, v_cache  updated in place; every other word is left untouched.
 * num_tokens == 0 is a no-op.
 */
pa_status_t pa_reshape_and_cache(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                 int32_t head_dim, const void *key, const void *value,
                                 void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                 int32_t num_tokens, void *stream);

/*
 * pa_copy_blocks -- copy-on-write of shared blocks ([MEM] 机制 2：写时复制: samples that share a
 * prompt's blocks by reference count get a private copy where they diverge).
 *   block_mapping [num_pairs][2] int32 (src, dst): the WHOLE block src -- all 16 slots, all kv heads
 *                 -- is copied to block dst, in both caches, bit for bit. Destinations must be
 *                 distinct and no destination may also be a source (the order of the copies is then
 *                 irrelevant).
 * dtype may be PA_DTYPE_FP8_E4M3 (caches of E4M3 codes: a block is then half as many bytes).
 * num_pairs == 0 is a no-op.
 */
pa_status_t pa_copy_blocks(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, void *k_cache, void *v_cache,
                           const int32_t *block_mapping, int32_t num_pairs, void *stream);

/*
 * Bytes of device workspace pa_decode needs for these sizes (0 when no partial results are kept:
 * partition_size == 0 or max_seq_len <= partition_size).
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_seq_len, int32_t partition_size);

/*
 * pa_decode -- one query token per sequence attends its whole paged history.
 * [PD] §3.1: the step's query q_t attends K_{1:t}, V_{1:t}, which already hold its own k_t, v_t
 * (write them first with pa_reshape_and_cache); [MEM] Attention 计算时的 Block 映射: position i is
 * read from block block_tables[s][i / 16] at offset i % 16; [PD] §3.4: GQA groups.
 *   out, query    [num_seqs][num_q_heads][head_dim]; out[s][h] = softmax(scale * q K^T) V over
 *                 positions 0 .. seq_lens[s]-1 of kv head h / group; a zero length gives zeros.
 *   block_tables  [num_seqs][max_blocks_per_seq] int32; only entries < ceil(seq_lens[s] / 16) are
 *                 read (padding such as -1 is never read).
 *   seq_lens      [num_seqs] int32, counting the token being decoded.
 *   max_seq_len   a host-side upper bound on seq_lens (sizes the launch); <= 16 * max_blocks_per_seq.
 *   partition_size  0: one pass per (sequence, kv head). Otherwise a multiple of 16 (at most 1024):
 *                 each sequence is cut into parts of that many tokens (head groups of 3 or more:
 *                 slots of 4 * partition_size tokens, each split evenly over four waves in 32-token
 *                 steps), processed in parallel, and merged by rescaling with the parts' maxima and
 *                 sums of exponentials ([OV] §9 (4)). It changes only the fp32 rounding.
 *   workspace     device scratch of at least pa_decode_workspace_size(...) bytes (may be NULL when
 *                 that is 0); its contents are overwritten.
 * `out` must not alias any input.
 */
pa_status_t pa_decode(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                      int32_t head_dim, void *out, const void *query, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                      int32_t max_seq_len, int32_t num_q_heads, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It takes no workspace and
 * allocates nothing: the split-K partial results go to a static scratch array inside this library
 * (PA_DECODE_SCRATCH_BYTES, 64 MiB), one copy on every GPU the library runs on, held from its
 * first use there until the process ends. Its address on a GPU is looked up once (the first call
 * on that GPU, for the device that owns `stream`; the current device for the null stream).
 * Arguments, results and errors are those of pa_decode (16-bit caches), with two more rules:
 *   - the partial results of these sizes, num_seqs * num_q_heads * slots * (head_dim + 2) fp32
 *     values (slots = ceil(ceil(max_seq_len / partition_size) / w), w = 4 for head groups of 3 or
 *     more, else 1; none when unsplit), must fit PA_DECODE_SCRATCH_BYTES, else PA_ERR_WORKSPACE
 *     before anything is enqueued;
 *   - every call on one GPU shares its scratch: calls that overlap in time on one GPU (different
 *     streams, or threads without ordering) race and give unspecified output. Calls ordered on one
 *     stream are safe. Nothing in the scratch needs to start at zero: each call writes every
 *     partial it reads.
 */
#define PA_DECODE_SCRATCH_BYTES ((size_t)64 << 20)

pa_status_t pa_decode_noalloc(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                              int32_t head_dim, void *out, const void *query, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *seq_lens,
                              int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                              float scale, int32_t partition_size, void *stream);

/*
 * pa_decode_shared_prefix -- pa_decode for batches whose sequences share prompt blocks, reading
 * each shared block once. [MEM] 机制 2：写时复制: parallel samples of one prompt share its
 * physical blocks (reference-counted) and diverge into private blocks; [V1] §2.2: shared prefixes.
 * Group g is the consecutive sequences group_starts[g] .. group_starts[g+1]-1 (group_starts[0] = 0;
 * sequences from group_starts[num_groups] on belong to no group). prefix_lens[s] (a multiple of 16)
 * is the number of leading positions whose blocks every member of s's group holds in common: the
 * same for all members, <= seq_lens of every member, and 0 for a sequence in no group. The
 * caller guarantees that those table entries are equal across the members.
 * Per (group, kv head) the shared positions are attended once for all members' queries, each
 * sequence's remaining positions by itself, and the parts are merged by rescaling with their
 * maxima and sums of exponentials ([OV] §9 (4)). out equals pa_decode's definition.
 *   Arguments as in pa_decode, plus group_starts [num_groups + 1], prefix_lens [num_seqs],
 *   max_group_size (>= every group's size, <= 64), max_prefix_len (>= every prefix_lens) and
 *   max_own_len: an upper bound on every sequence's own range, seq_lens[s] - prefix_lens[s]
 *   (<= 0: max_seq_len). It sizes the launch of the own-range units: a tight bound skips launching
 *   units past every own range, and when every own range fits one part of head groups of 1 or 2,
 *   each own unit also folds in its row's shared-prefix partials and writes the output (no merge
 *   pass). Own ranges longer than it give unspecified output, never a fault.
 *   partition_size must be a multiple of 16 in [16, 1024]; workspace of at least
 *   pa_decode_shared_prefix_workspace_size(...) bytes.
 */
size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t head_dim, int32_t max_seq_len,
                                              int32_t max_prefix_len, int32_t partition_size);

pa_status_t pa_decode_shared_prefix(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                    int32_t head_dim, void *out, const void *query,
                                    const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *seq_lens, int32_t num_seqs,
                                    int32_t max_seq_len, const int32_t *group_starts,
                                    const int32_t *prefix_lens, int32_t num_groups,
                                    int32_t max_group_size, int32_t max_prefix_len,
                                    int32_t max_own_len, int32_t num_q_heads, float scale,
                                    int32_t partition_size, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * pa_prefill_chunk -- causal attention of prefill chunks over their paged context.
 * [PD] §5.4: a long prompt is processed in chunks; a chunk attends the already-cached context and
 * the earlier part of itself. [PD] §1.1: causal order.
 *   query, out    [total_q][num_q_heads][head_dim]. Sequence s owns rows cu_q_lens[s] ..
 *                 cu_q_lens[s+1]-1, which are its last q_len_s = cu_q_lens[s+1] - cu_q_lens[s]
 *                 positions: row i of the chunk is at position p = seq_lens[s] - q_len_s + i and
 *                 attends positions 0..p inclusive. The chunk's own keys and values must already be
 *                 in the cache (pa_reshape_and_cache).
 *   cu_q_lens     [num_seqs + 1] int32, non-decreasing from 0 to total_q.
 *   seq_lens      [num_seqs] int32 (context including the chunk); block_tables as in pa_decode.
 *   max_q_len     a host-side upper bound on q_len_s (sizes the launch).
 * Rows whose position would be negative (q_len_s > seq_lens[s]) are written as zeros.
 */
pa_status_t pa_prefill_chunk(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                             int32_t head_dim, void *out, const void *query,
                             const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *seq_lens, const int32_t *cu_q_lens,
                             int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                             int32_t num_q_heads, float scale, void *stream);

/*
 * Bytes of the optional pa_prefill_chunk_fp8 workspace: a 16-bit copy of num_seqs *
 * max_blocks_per_seq blocks of both caches (2 * 16 * num_kv_heads * head_dim bytes per block and
 * cache, each cache's region rounded up to 256 bytes); 0 for non-positive arguments.
 */
size_t pa_prefill_chunk_fp8_workspace_size(int32_t num_seqs, int32_t max_blocks_per_seq,
                                           int32_t num_kv_heads, int32_t head_dim);

/*
 * pa_prefill_chunk_fp8 -- pa_prefill_chunk over E4M3 caches ([V1] §4.4 with [PD] §5.4): keys and
 * values are read as code value times k_scale / v_scale; query and out are of `dtype` (F16 or
 * BF16); layouts, the other arguments and errors as in pa_prefill_chunk.
 *   workspace     NULL, or device memory of at least pa_prefill_chunk_fp8_workspace_size(num_seqs,
 *                 max_blocks_per_seq, num_kv_heads, head_dim) bytes, 256-byte aligned (else
 *                 PA_ERR_WORKSPACE / PA_ERR_INVALID_ARG before anything is enqueued; its contents
 *                 are overwritten). With a workspace, every block of the context of each sequence
 *                 is first widened exactly to the 16-bit type (one pass over the E4M3 codes) and
 *                 the 16-bit kernel then reads it by direct-to-LDS loads, which is faster for a
 *                 chunk that is compute-bound; results are bit-identical to the path without one,
 *                 which converts the codes inside the tile loop. num_seqs * max_blocks_per_seq
 *                 must not exceed 2^31 - 1.
 */
pa_status_t pa_prefill_chunk_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                 int32_t head_dim, void *out, const void *query,
                                 const void *k_cache, const void *v_cache,
                                 const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *seq_lens, const int32_t *cu_q_lens,
                                 int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                 int32_t num_q_heads, float scale, float k_scale, float v_scale,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_prefill_chunk_tree -- pa_prefill_chunk for chunks that hold a tree of drafted tokens.
 * [V1] §5.3: a draft tree (EAGLE) is checked by the target model in one pass, every drafted token
 * seeing the context and the drafted tokens on its own path from the root; [PD] §5.4: the k drafts
 * are verified together. The chunk rows of sequence s are the drafted tokens, stored at positions
 * first_s .. seq_lens[s]-1 (first_s = seq_lens[s] - q_len_s) in tree order (a node after its
 * parent). Row i (position first_s + i) attends every position 0..first_s-1 and chunk row j
 * exactly when j <= i and bit j of tree_mask[cu_q_lens[s] + i] is set -- the mask of a node is
 * usually its ancestors and itself. A row that attends no position is written as zeros.
 *   tree_mask     [total_q] uint64, device memory, 8-byte aligned; bits j > i are ignored.
 *   max_q_len     at most 64 (PA_ERR_INVALID_ARG otherwise); q_len_s <= max_q_len and
 *                 q_len_s <= seq_lens[s] are the caller's contract.
 * Everything else -- layouts, the other arguments, errors -- as in pa_prefill_chunk.
 */
pa_status_t pa_prefill_chunk_tree(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                  int32_t head_dim, void *out, const void *query,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *seq_lens, const int32_t *cu_q_lens,
                                  const uint64_t *tree_mask, int32_t num_seqs, int32_t total_q,
                                  int32_t max_q_len, int32_t num_q_heads, float scale,
                                  void *stream);

/*
 * pa_reshape_and_cache_fp8 -- pa_reshape_and_cache into E4M3 caches ([V1] §4.4).
 * key and value are [num_tokens][num_kv_heads][head_dim] elements of `dtype` (F16 or BF16). The
 * byte written for element x is the E4M3 code of x / k_scale (keys) or x / v_scale (values): the
 * quotient rounded to float32, then to the nearest E4M3 value with ties to the even code;
 * magnitudes of 448 and more (infinities included) saturate to 448, and NaN gives code 0x7F with
 * x's sign. slot_mapping as in pa_reshape_and_cache. k_scale and v_scale: finite and positive.
 */
pa_status_t pa_reshape_and_cache_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                     int32_t head_dim, const void *key, const void *value,
                                     void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                     int32_t num_tokens, float k_scale, float v_scale,
                                     void *stream);

/*
 * pa_decode_fp8 -- pa_decode over E4M3 caches ([V1] §4.4): keys and values are read as code value
 * times k_scale / v_scale, everything else as in pa_decode (query and out of `dtype`, the same
 * workspace size function, partition_size rules and errors). Head groups of any size run.
 */
pa_status_t pa_decode_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, void *out, const void *query, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                          int32_t max_seq_len, int32_t num_q_heads, float scale, float k_scale,
                          float v_scale, int32_t partition_size, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * pa_decode_shared_prefix_fp8 -- pa_decode_shared_prefix over E4M3 caches ([V1] §4.4 with §2.2):
 * keys and values are read as code value times k_scale / v_scale; groups, prefix lengths, the
 * workspace size function (pa_decode_shared_prefix_workspace_size), partition_size rules and
 * errors are those of pa_decode_shared_prefix. out equals pa_decode_fp8's result for the same
 * sequences: the shared blocks are read once per group instead of once per member.
 */
pa_status_t pa_decode_shared_prefix_fp8(pa_dtype_t dtype, int32_t num_blocks,
                                        int32_t num_kv_heads, int32_t head_dim, void *out,
                                        const void *query, const void *k_cache,
                                        const void *v_cache, const int32_t *block_tables,
                                        int32_t max_blocks_per_seq, const int32_t *seq_lens,
                                        int32_t num_seqs, int32_t max_seq_len,
                                        const int32_t *group_starts, const int32_t *prefix_lens,
                                        int32_t num_groups, int32_t max_group_size,
                                        int32_t max_prefix_len, int32_t max_own_len,
                                        int32_t num_q_heads, float scale, float k_scale,
                                        float v_scale, int32_t partition_size, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * pa_decode_multi -- a few query rows per sequence (multi-token decode), read like a decode.
 * [PD] §5.4: the k drafts of a speculative step are verified by one pass of the target model;
 * [V1] §5.3: a draft tree (EAGLE) is verified the same way. The rows of sequence s are
 * cu_q_lens[s] .. cu_q_lens[s+1]-1 of query and out, at positions first_s .. seq_lens[s]-1
 * (first_s = seq_lens[s] - q_len_s). Row i attends positions 0..first_s-1 and the rows' own
 * positions first_s + j for j <= i; with tree_mask, only those j whose bit j of
 * tree_mask[cu_q_lens[s] + i] is set. out equals pa_prefill_chunk's (pa_prefill_chunk_tree's with
 * a mask) for the same rows; a row that attends no position is written as zeros.
 * Each kv head's context is read once per 32 (row, query head) pairs, on MFMA, split into parts of
 * partition_size tokens merged by rescaling with their maxima and sums of exponentials, as in
 * pa_decode ([OV] §9 (4)). The chunk kernel of pa_prefill_chunk instead reads it once per
 * workgroup of 256 pairs (128 where the block tables span at most 2048 tokens), which few rows
 * leave mostly empty: this call is the faster one up to 32 pairs per kv head (max_q_len *
 * num_q_heads / num_kv_heads), the two are even at 64.
 *   query, out    [total_q][num_q_heads][head_dim] of `dtype` (F16 or BF16); out must not alias
 *                 an input.
 *   cu_q_lens     [num_seqs + 1] int32, cu_q_lens[0] = 0, non-decreasing, cu_q_lens[num_seqs] =
 *                 total_q; q_len_s <= max_q_len and q_len_s <= seq_lens[s] are the caller's
 *                 contract (rows past max_q_len are not written).
 *   tree_mask     NULL (causal rows) or [total_q] uint64, device memory, 8-byte aligned; bits
 *                 j > i are ignored.
 *   max_q_len     1..16 (PA_ERR_INVALID_ARG otherwise).
 *   max_seq_len   an upper bound on seq_lens (sizes the launch); <= 16 * max_blocks_per_seq.
 *   partition_size, workspace: as in pa_decode, with a workspace of at least
 *                 pa_decode_multi_workspace_size(...) bytes (0 when unsplit).
 * The other arguments, layouts and errors are those of pa_decode.
 */
size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_seq_len,
                                      int32_t partition_size);

pa_status_t pa_decode_multi(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                            int32_t head_dim, void *out, const void *query, const void *k_cache,
                            const void *v_cache, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens,
                            const int32_t *cu_q_lens, const uint64_t *tree_mask, int32_t num_seqs,
                            int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                            int32_t num_q_heads, float scale, int32_t partition_size,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_multi_fp8 -- pa_decode_multi over E4M3 caches ([V1] §4.4): keys and values are read
 * as code value times k_scale / v_scale (finite, positive); everything else as in pa_decode_multi.
 */
pa_status_t pa_decode_multi_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                int32_t head_dim, void *out, const void *query,
                                const void *k_cache, const void *v_cache,
                                const int32_t *block_tables, int32_t max_blocks_per_seq,
                                const int32_t *seq_lens, const int32_t *cu_q_lens,
                                const uint64_t *tree_mask, int32_t num_seqs, int32_t total_q,
                                int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                                float scale, float k_scale, float v_scale,
                                int32_t partition_size, void *workspace, size_t workspace_bytes,
                                void *stream);

/* Static text for a status code. */
const char *pa_status_string(pa_status_t status);

/* The calling thread's last error message ("" when the last call succeeded). */
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
