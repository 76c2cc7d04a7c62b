// block_manager.cpp -- the host-side block manager of include/pa_block_manager.h.
//
// Pool: every block has a reference count; blocks with count 0 sit in one doubly linked free
// queue threaded through `prev`/`next` arrays (sentinel = index num_blocks), so taking the head,
// appending at the tail and unlinking a block from the middle are all O(1) ([V1] §1.2).
// Prefix cache ([V1] §2.2, §2.3): a full block whose token ids are known is entered in a hash map
// under a 64-bit hash chained over the sequence's blocks; the block keeps that hash, its parent's
// hash and its 16 ids so that a lookup can check what it found. A cached block whose count drops
// to 0 stays in the map while it waits in the free queue; it leaves the map only when allocation
// takes it from the head of the queue.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_block_manager.h"
#include "pa_internal.h"

using pa::fail;
using pa::ok;

namespace {

constexpr int32_t B = PA_BLOCK_SIZE;
constexpr uint64_t kRootHash = 0x243F6A8885A308D3ull;  // parent hash of a sequence's first block

// splitmix64's output function: a bijective 64-bit mix.
inline uint64_t mix64(uint64_t x)
{
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 31;
    return x;
}

// Hash of a block's contents given its parent's hash: the chain covers every token id from
// position 0 to the end of the block.
uint64_t chain_hash(uint64_t parent, const int32_t *ids)
{
    uint64_t h = mix64(parent ^ 0x9E3779B97F4A7C15ull);
    for (int i = 0; i < B; ++i)
        h = mix64(h + (uint64_t)(uint32_t)ids[i] + 0x9E3779B97F4A7C15ull * (uint64_t)(i + 1));
    return h;
}

struct Sequence {
    std::vector<int32_t> blocks;   // block table, logical order
    int32_t num_tokens = 0;
    bool ids_known = true;         // every token so far came with its id
    std::vector<uint64_t> hashes;  // chain hash of each full block (while ids_known)
    std::vector<int32_t> tail;     // ids of the tokens in the partly filled last block
};

}  // namespace

struct pa_block_manager {
    int32_t n = 0;
    bool prefix_caching = false;
    std::vector<int32_t> ref_cnt;
    std::vector<int32_t> prev, next;  // free-queue links, size n + 1; n is the sentinel
    std::vector<uint8_t> in_queue;
    int32_t num_free = 0;
    std::vector<uint8_t> cached;
    std::vector<uint64_t> hash, parent_hash;
    std::vector<int32_t> ids;  // [n][16] ids of cached blocks
    std::unordered_map<uint64_t, int32_t> by_hash;
    std::unordered_map<int64_t, Sequence> seqs;

    void push_tail(int32_t b)
    {
        int32_t last = prev[n];
        next[last] = b;
        prev[b] = last;
        next[b] = n;
        prev[n] = b;
        in_queue[b] = 1;
        ++num_free;
    }
    void unlink(int32_t b)
    {
        next[prev[b]] = next[b];
        prev[next[b]] = prev[b];
        in_queue[b] = 0;
        --num_free;
    }
    void uncache(int32_t b)
    {
        if (!cached[b])
            return;
        auto it = by_hash.find(hash[b]);
        if (it != by_hash.end() && it->second == b)
            by_hash.erase(it);
        cached[b] = 0;
    }
    // Take the head of the free queue for a new owner (evicting it from the prefix cache).
    int32_t take()
    {
        int32_t b = next[n];
        unlink(b);
        uncache(b);
        ref_cnt[b] = 1;
        return b;
    }
    void release(int32_t b)
    {
        if (--ref_cnt[b] == 0)
            push_tail(b);
    }
    // Enter full block b (its ids at `blk_ids`, chain hash h, parent hash ph) in the cache unless
    // a block with the same contents is already there.
    void register_block(int32_t b, uint64_t h, uint64_t ph, const int32_t *blk_ids)
    {
        if (cached[b] || by_hash.count(h))
            return;
        by_hash.emplace(h, b);
        cached[b] = 1;
        hash[b] = h;
        parent_hash[b] = ph;
        memcpy(&ids[(size_t)b * B], blk_ids, sizeof(int32_t) * B);
    }
    // The cached block holding these contents, or -1.
    int32_t lookup(uint64_t h, uint64_t ph, const int32_t *blk_ids) const
    {
        auto it = by_hash.find(h);
        if (it == by_hash.end())
            return -1;
        int32_t b = it->second;
        if (!cached[b] || parent_hash[b] != ph ||
            memcmp(&ids[(size_t)b * B], blk_ids, sizeof(int32_t) * B) != 0)
            return -1;
        return b;
    }
};

namespace {

pa_status_t find_seq(const pa_block_manager *bm, int64_t id, const Sequence **out)
{
    if (bm == nullptr)
        return fail(PA_ERR_INVALID_ARG, "block manager is NULL");
    auto it = bm->seqs.find(id);
    if (it == bm->seqs.end())
        return fail(PA_ERR_INVALID_ARG, "no live sequence %lld", (long long)id);
    *out = &it->second;
    return PA_OK;
}

pa_status_t find_seq(pa_block_manager *bm, int64_t id, Sequence **out)
{
    const Sequence *s = nullptr;
    pa_status_t st = find_seq((const pa_block_manager *)bm, id, &s);
    *out = const_cast<Sequence *>(s);
    return st;
}

}  // namespace

extern "C" {

pa_status_t pa_bm_create(int32_t num_blocks, const int32_t *free_order, int32_t prefix_caching,
                         pa_block_manager **out)
{
    if (out == nullptr)
        return fail(PA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || num_blocks > INT32_MAX / B)
        return fail(PA_ERR_INVALID_ARG, "num_blocks %d outside [1, %d]", num_blocks,
                    INT32_MAX / B);
    pa_block_manager *bm = new (std::nothrow) pa_block_manager();
    if (bm == nullptr)
        return fail(PA_ERR_INVALID_ARG, "out of host memory");
    try {
        bm->n = num_blocks;
        bm->prefix_caching = prefix_caching != 0;
        bm->ref_cnt.assign(num_blocks, 0);
        bm->prev.assign(num_blocks + 1, num_blocks);
        bm->next.assign(num_blocks + 1, num_blocks);
        bm->in_queue.assign(num_blocks, 0);
        bm->cached.assign(num_blocks, 0);
        bm->hash.assign(num_blocks, 0);
        bm->parent_hash.assign(num_blocks, 0);
        if (bm->prefix_caching)
            bm->ids.assign((size_t)num_blocks * B, 0);
    } catch (const std::bad_alloc &) {
        delete bm;
        return fail(PA_ERR_INVALID_ARG, "out of host memory for %d blocks", num_blocks);
    }
    for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t b = free_order ? free_order[i] : i;
        if (b < 0 || b >= num_blocks || bm->in_queue[b]) {
            delete bm;
            return fail(PA_ERR_INVALID_ARG, "free_order is not a permutation of 0..%d (entry %d)",
                        num_blocks - 1, i);
        }
        bm->push_tail(b);
    }
    *out = bm;
    return ok();
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

pa_status_t pa_bm_add_sequence(pa_block_manager *bm, int64_t seq_id)
{
    if (bm == nullptr)
        return fail(PA_ERR_INVALID_ARG, "block manager is NULL");
    if (bm->seqs.count(seq_id))
        return fail(PA_ERR_INVALID_ARG, "sequence %lld is already live", (long long)seq_id);
    bm->seqs.emplace(seq_id, Sequence());
    return ok();
}

pa_status_t pa_bm_match_prefix(pa_block_manager *bm, int64_t seq_id, const int32_t *token_ids,
                               int32_t num_tokens, int32_t *num_cached_tokens)
{
    Sequence *s = nullptr;
    pa_status_t st = find_seq(bm, seq_id, &s);
    if (st != PA_OK)
        return st;
    if (num_cached_tokens == nullptr)
        return fail(PA_ERR_INVALID_ARG, "num_cached_tokens is NULL");
    if (num_tokens < 0)
        return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
    if (num_tokens > 0 && token_ids == nullptr)
        return fail(PA_ERR_INVALID_ARG, "token_ids is NULL");
    if (s->num_tokens != 0)
        return fail(PA_ERR_INVALID_ARG, "sequence %lld already holds %d tokens", (long long)seq_id,
                    s->num_tokens);
    *num_cached_tokens = 0;
    if (!bm->prefix_caching || num_tokens <= 1)
        return ok();
    const int32_t max_hit = (num_tokens - 1) / B;
    uint64_t parent = kRootHash;
    for (int32_t j = 0; j < max_hit; ++j) {
        const int32_t *blk = token_ids + (size_t)j * B;
        uint64_t h = chain_hash(parent, blk);
        int32_t b = bm->lookup(h, parent, blk);
        if (b < 0)
            break;
        if (bm->ref_cnt[b] == 0)
            bm->unlink(b);
        ++bm->ref_cnt[b];
        s->blocks.push_back(b);
        s->hashes.push_back(h);
        parent = h;
    }
    s->num_tokens = (int32_t)s->blocks.size() * B;
    *num_cached_tokens = s->num_tokens;
    return ok();
}

pa_status_t pa_bm_allocate_slots(pa_block_manager *bm, int64_t seq_id, const int32_t *token_ids,
                                 int32_t num_tokens, int32_t *slots, int32_t cow_pair[2])
{
    Sequence *s = nullptr;
    pa_status_t st = find_seq(bm, seq_id, &s);
    if (st != PA_OK)
        return st;
    if (num_tokens < 0)
        return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
    if (cow_pair == nullptr || (num_tokens > 0 && slots == nullptr))
        return fail(PA_ERR_INVALID_ARG, "slots or cow_pair is NULL");
    cow_pair[0] = cow_pair[1] = -1;
    if (num_tokens == 0)
        return ok();
    const int64_t L0 = s->num_tokens, L1 = L0 + num_tokens;
    if (L1 > (int64_t)INT32_MAX)
        return fail(PA_ERR_INVALID_ARG, "sequence length %lld overflows int32", (long long)L1);
    const bool cow = (L0 % B) != 0 && bm->ref_cnt[s->blocks.back()] > 1;
    const int64_t fresh = (L1 + B - 1) / B - (int64_t)s->blocks.size() + (cow ? 1 : 0);
    if (fresh > bm->num_free)
        return fail(PA_ERR_NO_BLOCKS, "sequence %lld needs %lld free blocks, the queue holds %d",
                    (long long)seq_id, (long long)fresh, bm->num_free);

    if (cow) {
        int32_t shared = s->blocks.back();
        int32_t copy = bm->take();
        --bm->ref_cnt[shared];  // still >= 1: other holders keep it
        s->blocks.back() = copy;
        cow_pair[0] = shared;
        cow_pair[1] = copy;
    }
    const bool track = bm->prefix_caching && s->ids_known && token_ids != nullptr;
    for (int32_t i = 0; i < num_tokens; ++i) {
        const int64_t pos = L0 + i;
        const int32_t lb = (int32_t)(pos / B);
        if (lb == (int32_t)s->blocks.size())
            s->blocks.push_back(bm->take());
        slots[i] = s->blocks[lb] * B + (int32_t)(pos % B);
        if (track) {
            s->tail.push_back(token_ids[i]);
            if ((pos + 1) % B == 0) {
                uint64_t ph = s->hashes.empty() ? kRootHash : s->hashes.back();
                uint64_t h = chain_hash(ph, s->tail.data());
                bm->register_block(s->blocks[lb], h, ph, s->tail.data());
                s->hashes.push_back(h);
                s->tail.clear();
            }
        }
    }
    if (!track) {
        s->ids_known = false;
        s->tail.clear();
    }
    s->num_tokens = (int32_t)L1;
    return ok();
}

pa_status_t pa_bm_fork(pa_block_manager *bm, int64_t parent_id, int64_t child_id)
{
    Sequence *p = nullptr;
    pa_status_t st = find_seq(bm, parent_id, &p);
    if (st != PA_OK)
        return st;
    if (bm->seqs.count(child_id))
        return fail(PA_ERR_INVALID_ARG, "sequence %lld is already live", (long long)child_id);
    Sequence child = *p;  // copied before the emplace, which may rehash
    for (int32_t b : child.blocks)
        ++bm->ref_cnt[b];
    bm->seqs.emplace(child_id, std::move(child));
    return ok();
}

pa_status_t pa_bm_free(pa_block_manager *bm, int64_t seq_id)
{
    Sequence *s = nullptr;
    pa_status_t st = find_seq(bm, seq_id, &s);
    if (st != PA_OK)
        return st;
    for (auto it = s->blocks.rbegin(); it != s->blocks.rend(); ++it)
        bm->release(*it);
    bm->seqs.erase(seq_id);
    return ok();
}

pa_status_t pa_bm_sequence_info(const pa_block_manager *bm, int64_t seq_id, int32_t *num_tokens,
                                int32_t *num_blocks)
{
    const Sequence *s = nullptr;
    pa_status_t st = find_seq(bm, seq_id, &s);
    if (st != PA_OK)
        return st;
    if (num_tokens)
        *num_tokens = s->num_tokens;
    if (num_blocks)
        *num_blocks = (int32_t)s->blocks.size();
    return ok();
}

pa_status_t pa_bm_block_tables(const pa_block_manager *bm, const int64_t *seq_ids,
                               int32_t num_seqs, int32_t max_blocks_per_seq, int32_t *out)
{
    if (bm == nullptr)
        return fail(PA_ERR_INVALID_ARG, "block manager is NULL");
    if (num_seqs < 0 || max_blocks_per_seq < 0)
        return fail(PA_ERR_INVALID_ARG, "num_seqs %d or max_blocks_per_seq %d < 0", num_seqs,
                    max_blocks_per_seq);
    if (num_seqs == 0)
        return ok();
    if (seq_ids == nullptr || (out == nullptr && max_blocks_per_seq > 0))
        return fail(PA_ERR_INVALID_ARG, "seq_ids or out is NULL");
    for (int32_t i = 0; i < num_seqs; ++i) {  // check everything before writing anything
        const Sequence *s = nullptr;
        pa_status_t st = find_seq(bm, seq_ids[i], &s);
        if (st != PA_OK)
            return st;
        if ((int32_t)s->blocks.size() > max_blocks_per_seq)
            return fail(PA_ERR_INVALID_ARG, "sequence %lld holds %d blocks > max_blocks_per_seq %d",
                        (long long)seq_ids[i], (int)s->blocks.size(), max_blocks_per_seq);
    }
    for (int32_t i = 0; i < num_seqs; ++i) {
        const Sequence &s = bm->seqs.find(seq_ids[i])->second;
        int32_t *row = out + (size_t)i * max_blocks_per_seq;
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        std::fill(row + s.blocks.size(), row + max_blocks_per_seq, -1);
    }
    return ok();
}

int32_t pa_bm_num_free_blocks(const pa_block_manager *bm) { return bm ? bm->num_free : 0; }

int32_t pa_bm_free_queue(const pa_block_manager *bm, int32_t *out, int32_t capacity)
{
    if (bm == nullptr || (out == nullptr && capacity > 0))
        return -1;
    int32_t k = 0;
    for (int32_t b = bm->next[bm->n]; b != bm->n && k < capacity; b = bm->next[b])
        out[k++] = b;
    return k;
}

pa_status_t pa_bm_block_state(const pa_block_manager *bm, int32_t block, int32_t *ref_cnt,
                              int32_t *is_cached)
{
    if (bm == nullptr || ref_cnt == nullptr)
        return fail(PA_ERR_INVALID_ARG, "block manager or ref_cnt is NULL");
    if (block < 0 || block >= bm->n)
        return fail(PA_ERR_INVALID_ARG, "block %d outside [0, %d)", block, bm->n);
    *ref_cnt = bm->ref_cnt[block];
    if (is_cached)
        *is_cached = bm->cached[block];
    return ok();
}

}  // extern "C"
