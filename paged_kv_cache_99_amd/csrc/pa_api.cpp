// pa_api.cpp -- the C ABI declared in include/pa.h: host-side argument checks, workspace layout
// and dispatch to the kernel launchers. Nothing here reads device memory or synchronises.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "pa.h"
#include "pa_internal.h"

namespace {
thread_local char g_error[512] = "";
}  // namespace

namespace pa {

pa_status_t fail(pa_status_t s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return s;
}

pa_status_t ok()
{
    g_error[0] = '\0';
    return PA_OK;
}

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, ...)                                    \
    do {                                                      \
        if (!(cond))                                          \
            return fail(PA_ERR_INVALID_ARG, __VA_ARGS__);     \
    } while (0)

#define REQUIRE_PTR(p, name)                                                              \
    do {                                                                                  \
        REQUIRE((p) != nullptr, "%s is NULL", name);                                      \
        REQUIRE(aligned16(p), "%s is not 16-byte aligned", name);                         \
    } while (0)

// allow_fp8: dtype may name E4M3 caches (an operation that only moves cache bytes).
pa_status_t check_cache(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, pa::CacheDims *c, bool allow_fp8 = false)
{
    if (allow_fp8)
        REQUIRE(dtype == PA_DTYPE_F16 || dtype == PA_DTYPE_BF16 || dtype == PA_DTYPE_FP8_E4M3,
                "dtype %d is not F16, BF16 or FP8_E4M3", (int)dtype);
    else
        REQUIRE(dtype == PA_DTYPE_F16 || dtype == PA_DTYPE_BF16, "dtype %d is not F16 or BF16",
                (int)dtype);
    REQUIRE(num_blocks >= 0, "num_blocks %d < 0", num_blocks);
    REQUIRE(num_kv_heads > 0, "num_kv_heads %d <= 0", num_kv_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d: kernels exist for 64 and 128", head_dim);
    REQUIRE((int64_t)num_blocks * num_kv_heads * PA_BLOCK_SIZE * head_dim < ((int64_t)1 << 40),
            "cache of %d blocks is too large", num_blocks);
    c->num_blocks = num_blocks;
    c->num_kv_heads = num_kv_heads;
    c->head_dim = head_dim;
    c->bf16 = dtype == PA_DTYPE_BF16;
    c->fp8 = dtype == PA_DTYPE_FP8_E4M3;
    return PA_OK;
}

bool good_scale(float x) { return x > 0.0f && x < 3.0e38f; }

pa_status_t launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int32_t parts_of(int32_t max_seq_len, int32_t partition_size)
{
    if (partition_size <= 0 || max_seq_len <= partition_size)
        return 0;
    return (max_seq_len + partition_size - 1) / partition_size;
}

}  // namespace

extern "C" {

const char *pa_status_string(pa_status_t status)
{
    switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: an argument failed its check";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: no kernel for this shape";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP launch failed";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free blocks in the pool";
    }
    return "unknown pa_status_t";
}

const char *pa_last_error(void) { return g_error; }

pa_status_t pa_reshape_and_cache(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                 int32_t head_dim, const void *key, const void *value,
                                 void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                 int32_t num_tokens, void *stream)
{
    pa::CacheDims c;
    pa_status_t s = check_cache(dtype, num_blocks, num_kv_heads, head_dim, &c);
    if (s != PA_OK)
        return s;
    REQUIRE(num_tokens >= 0, "num_tokens %d < 0", num_tokens);
    if (num_tokens == 0)
        return ok();
    REQUIRE_PTR(key, "key");
    REQUIRE_PTR(value, "value");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    REQUIRE(slot_mapping != nullptr, "slot_mapping is NULL");
    return launched(pa::launch_reshape_and_cache(c, key, value, k_cache, v_cache, slot_mapping,
                                                 num_tokens, (hipStream_t)stream),
                    "reshape_and_cache");
}

pa_status_t pa_reshape_and_cache_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                     int32_t head_dim, const void *key, const void *value,
                                     void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                     int32_t num_tokens, float k_scale, float v_scale,
                                     void *stream)
{
    pa::CacheDims c;
    pa_status_t s = check_cache(dtype, num_blocks, num_kv_heads, head_dim, &c);
    if (s != PA_OK)
        return s;
    c.fp8 = true;
    REQUIRE(num_tokens >= 0, "num_tokens %d < 0", num_tokens);
    REQUIRE(good_scale(k_scale) && good_scale(v_scale),
            "k_scale %g / v_scale %g is not a finite positive number", (double)k_scale,
            (double)v_scale);
    if (num_tokens == 0)
        return ok();
    REQUIRE_PTR(key, "key");
    REQUIRE_PTR(value, "value");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    REQUIRE(slot_mapping != nullptr, "slot_mapping is NULL");
    return launched(pa::launch_reshape_and_cache_fp8(c, key, value, k_cache, v_cache, slot_mapping,
                                                     num_tokens, k_scale, v_scale,
                                                     (hipStream_t)stream),
                    "reshape_and_cache_fp8");
}

pa_status_t pa_copy_blocks(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, void *k_cache, void *v_cache,
                           const int32_t *block_mapping, int32_t num_pairs, void *stream)
{
    pa::CacheDims c;
    pa_status_t s = check_cache(dtype, num_blocks, num_kv_heads, head_dim, &c, true);
    if (s != PA_OK)
        return s;
    REQUIRE(num_pairs >= 0, "num_pairs %d < 0", num_pairs);
    if (num_pairs == 0)
        return ok();
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    REQUIRE(block_mapping != nullptr, "block_mapping is NULL");
    return launched(pa::launch_copy_blocks(c, k_cache, v_cache, block_mapping, num_pairs,
                                           (hipStream_t)stream),
                    "copy_blocks");
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_seq_len, int32_t partition_size)
{
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0)
        return 0;
    const int32_t parts = parts_of(max_seq_len, partition_size);
    return (size_t)num_seqs * num_q_heads * parts * (head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

pa_status_t decode_call(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, void *out, const void *query, const void *k_cache,
                        const void *v_cache, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                        int32_t max_seq_len, int32_t num_q_heads, float scale,
                        int32_t partition_size, void *workspace, size_t workspace_bytes,
                        void *stream, bool fp8, float k_scale, float v_scale,
                        bool use_scratch = false)
{
    pa::CacheDims c;
    pa_status_t s = check_cache(dtype, num_blocks, num_kv_heads, head_dim, &c);
    if (s != PA_OK)
        return s;
    REQUIRE(num_seqs >= 0, "num_seqs %d < 0", num_seqs);
    REQUIRE(num_q_heads > 0 && num_q_heads % num_kv_heads == 0,
            "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
            num_kv_heads);
    REQUIRE(max_blocks_per_seq >= 0, "max_blocks_per_seq %d < 0", max_blocks_per_seq);
    REQUIRE(max_seq_len >= 0 && (int64_t)max_seq_len <= (int64_t)PA_BLOCK_SIZE * max_blocks_per_seq,
            "max_seq_len %d is outside [0, 16 * max_blocks_per_seq = %lld]", max_seq_len,
            (long long)PA_BLOCK_SIZE * max_blocks_per_seq);
    REQUIRE(partition_size >= 0 && partition_size % PA_BLOCK_SIZE == 0 && partition_size <= 1024,
            "partition_size %d is not 0 or a multiple of 16 up to 1024", partition_size);
    REQUIRE(scale > 0.0f && scale < 3.0e38f, "scale %g is not a finite positive number", (double)scale);
    if (fp8)
        REQUIRE(good_scale(k_scale) && good_scale(v_scale),
                "k_scale %g / v_scale %g is not a finite positive number", (double)k_scale,
                (double)v_scale);
    if (!pa::decode_supported(head_dim, num_q_heads / num_kv_heads))
        return fail(PA_ERR_UNSUPPORTED, "no decode kernel for head_dim %d, group %d", head_dim,
                    num_q_heads / num_kv_heads);
    if (num_seqs == 0)
        return ok();
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(query, "query");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    REQUIRE(block_tables != nullptr, "block_tables is NULL");
    REQUIRE(seq_lens != nullptr, "seq_lens is NULL");
    if (use_scratch) {
        // the library's static scratch instead of a caller's workspace: no allocation anywhere
        const size_t used = pa::decode_workspace_used(num_seqs, num_q_heads, num_kv_heads,
                                                      head_dim, max_seq_len, partition_size);
        if (used > pa::kDecodeScratchBytes)
            return fail(PA_ERR_WORKSPACE,
                        "partial results need %zu bytes, above the %zu-byte static scratch "
                        "(use pa_decode with a workspace, or a larger partition_size)",
                        used, pa::kDecodeScratchBytes);
        workspace = nullptr;
        if (used > 0) {
            const hipError_t e = pa::decode_scratch((hipStream_t)stream, &workspace);
            if (e != hipSuccess)
                return fail(PA_ERR_HIP, "decode scratch lookup: %s", hipGetErrorString(e));
        }
    } else {
        const size_t need =
            pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size);
        if (need > 0) {
            if (workspace == nullptr || workspace_bytes < need)
                return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed",
                            workspace_bytes, need);
            REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
        }
    }
    pa::DecodeLaunch d;
    d.c = c;
    d.out = out;
    d.query = query;
    d.k_cache = k_cache;
    d.v_cache = v_cache;
    d.block_tables = block_tables;
    d.max_blocks = max_blocks_per_seq;
    d.seq_lens = seq_lens;
    d.num_seqs = num_seqs;
    d.max_seq_len = max_seq_len;
    d.num_q_heads = num_q_heads;
    d.scale = scale;
    d.partition_size = partition_size;
    d.max_parts = parts_of(max_seq_len, partition_size);
    d.seq_starts = nullptr;
    d.group_starts = nullptr;
    d.num_groups = 0;
    d.max_group_size = 0;
    d.max_prefix_len = 0;
    d.workspace = workspace;
    d.fp8 = fp8;
    d.c.fp8 = fp8;
    d.k_scale = k_scale;
    d.v_scale = v_scale;
    return launched(pa::launch_decode(d, (hipStream_t)stream), fp8 ? "decode_fp8" : "decode");
}

}  // namespace

extern "C" {

pa_status_t pa_decode(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                      int32_t head_dim, void *out, const void *query, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                      int32_t max_seq_len, int32_t num_q_heads, float scale,
                      int32_t partition_size, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    return decode_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                       block_tables, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                       num_q_heads, scale, partition_size, workspace, workspace_bytes, stream,
                       false, 1.0f, 1.0f);
}

pa_status_t pa_decode_noalloc(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                              int32_t head_dim, void *out, const void *query, const void *k_cache,
                              const void *v_cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *seq_lens,
                              int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                              float scale, int32_t partition_size, void *stream)
{
    return decode_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                       block_tables, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                       num_q_heads, scale, partition_size, nullptr, 0, stream, false, 1.0f, 1.0f,
                       true);
}

pa_status_t pa_decode_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, void *out, const void *query, const void *k_cache,
                          const void *v_cache, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t num_seqs,
                          int32_t max_seq_len, int32_t num_q_heads, float scale, float k_scale,
                          float v_scale, int32_t partition_size, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    return decode_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                       block_tables, max_blocks_per_seq, seq_lens, num_seqs, max_seq_len,
                       num_q_heads, scale, partition_size, workspace, workspace_bytes, stream,
                       true, k_scale, v_scale);
}

size_t pa_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t head_dim, int32_t max_seq_len,
                                              int32_t max_prefix_len, int32_t partition_size)
{
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || partition_size <= 0 ||
        max_seq_len < 0 || max_prefix_len < 0)
        return 0;
    const int64_t own = max_seq_len > 0 ? (max_seq_len + partition_size - 1) / partition_size : 1;
    const int64_t pre = (max_prefix_len + partition_size - 1) / partition_size;
    return (size_t)num_seqs * num_q_heads * (size_t)(pre + own) * (head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

pa_status_t shared_prefix_call(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                               int32_t head_dim, void *out, const void *query,
                               const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *seq_lens, int32_t num_seqs, int32_t max_seq_len,
                               const int32_t *group_starts, const int32_t *prefix_lens,
                               int32_t num_groups, int32_t max_group_size,
                               int32_t max_prefix_len, int32_t max_own_len,
                               int32_t num_q_heads, float scale,
                               int32_t partition_size, void *workspace, size_t workspace_bytes,
                               void *stream, bool fp8, float k_scale, float v_scale)
{
    pa::CacheDims c;
    pa_status_t s = check_cache(dtype, num_blocks, num_kv_heads, head_dim, &c);
    if (s != PA_OK)
        return s;
    REQUIRE(num_seqs >= 0, "num_seqs %d < 0", num_seqs);
    REQUIRE(num_q_heads > 0 && num_q_heads % num_kv_heads == 0,
            "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
            num_kv_heads);
    REQUIRE(max_blocks_per_seq >= 0, "max_blocks_per_seq %d < 0", max_blocks_per_seq);
    REQUIRE(max_seq_len >= 0 && (int64_t)max_seq_len <= (int64_t)PA_BLOCK_SIZE * max_blocks_per_seq,
            "max_seq_len %d is outside [0, 16 * max_blocks_per_seq = %lld]", max_seq_len,
            (long long)PA_BLOCK_SIZE * max_blocks_per_seq);
    REQUIRE(partition_size > 0 && partition_size % PA_BLOCK_SIZE == 0 && partition_size <= 1024,
            "partition_size %d is not a multiple of 16 in [16, 1024]", partition_size);
    REQUIRE(scale > 0.0f && scale < 3.0e38f, "scale %g is not a finite positive number", (double)scale);
    REQUIRE(num_groups >= 0 && num_groups <= num_seqs, "num_groups %d is outside [0, num_seqs]",
            num_groups);
    REQUIRE(max_group_size >= 1 && max_group_size <= 64, "max_group_size %d is outside [1, 64]",
            max_group_size);
    REQUIRE(max_prefix_len >= 0 && max_prefix_len <= max_seq_len,
            "max_prefix_len %d is outside [0, max_seq_len]", max_prefix_len);
    if (fp8)
        REQUIRE(good_scale(k_scale) && good_scale(v_scale),
                "k_scale %g / v_scale %g is not a finite positive number", (double)k_scale,
                (double)v_scale);
    if (!pa::decode_supported(head_dim, num_q_heads / num_kv_heads))
        return fail(PA_ERR_UNSUPPORTED, "no decode kernel for head_dim %d, group %d", head_dim,
                    num_q_heads / num_kv_heads);
    if (num_seqs == 0)
        return ok();
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(query, "query");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    REQUIRE(block_tables != nullptr, "block_tables is NULL");
    REQUIRE(seq_lens != nullptr, "seq_lens is NULL");
    REQUIRE(prefix_lens != nullptr, "prefix_lens is NULL");
    REQUIRE(num_groups == 0 || group_starts != nullptr, "group_starts is NULL");
    const size_t need = pa_decode_shared_prefix_workspace_size(num_seqs, num_q_heads, head_dim,
                                                               max_seq_len, max_prefix_len,
                                                               partition_size);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
    REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
    // own parts per sequence: enough for the longest own range (positions after the shared prefix)
    const int32_t own_len =
        max_own_len > 0 && max_own_len < max_seq_len ? max_own_len : max_seq_len;
    const int32_t own = own_len > 0 ? (own_len + partition_size - 1) / partition_size : 1;
    pa::DecodeLaunch d;
    d.c = c;
    d.out = out;
    d.query = query;
    d.k_cache = k_cache;
    d.v_cache = v_cache;
    d.block_tables = block_tables;
    d.max_blocks = max_blocks_per_seq;
    d.seq_lens = seq_lens;
    d.num_seqs = num_seqs;
    d.max_seq_len = max_seq_len;
    d.num_q_heads = num_q_heads;
    d.scale = scale;
    d.partition_size = partition_size;
    d.max_parts = own;
    d.seq_starts = prefix_lens;
    d.group_starts = num_groups > 0 ? group_starts : nullptr;
    d.num_groups = num_groups;
    d.max_group_size = max_group_size;
    d.max_prefix_len = max_prefix_len;
    d.max_own_len = own_len;
    if (d.group_starts == nullptr) {
        // no groups: a plain split decode (every prefix length must then be 0)
        d.seq_starts = nullptr;
        d.max_prefix_len = 0;
    }
    d.workspace = workspace;
    d.fp8 = fp8;
    d.c.fp8 = fp8;
    d.k_scale = k_scale;
    d.v_scale = v_scale;
    return launched(pa::launch_decode(d, (hipStream_t)stream),
                    fp8 ? "decode_shared_prefix_fp8" : "decode_shared_prefix");
}

}  // namespace

extern "C" {

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
                                    size_t workspace_bytes, void *stream)
{
    return shared_prefix_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache,
                              v_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                              max_seq_len, group_starts, prefix_lens, num_groups, max_group_size,
                              max_prefix_len, max_own_len, num_q_heads, scale, partition_size,
                              workspace, workspace_bytes, stream, false, 1.0f, 1.0f);
}

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
                                        size_t workspace_bytes, void *stream)
{
    return shared_prefix_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache,
                              v_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                              max_seq_len, group_starts, prefix_lens, num_groups, max_group_size,
                              max_prefix_len, max_own_len, num_q_heads, scale, partition_size,
                              workspace, workspace_bytes, stream, true, k_scale, v_scale);
}

}  // extern "C"

namespace {

pa_status_t prefill_call(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, void *out, const void *query, const void *k_cache,
                         const void *v_cache, const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *seq_lens,
                         const int32_t *cu_q_lens, const uint64_t *tree_mask, bool tree,
                         int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                         int32_t num_q_heads, float scale, void *stream, bool fp8 = false,
                         float k_scale = 1.0f, float v_scale = 1.0f, void *workspace = nullptr,
                         size_t workspace_bytes = 0)
{
    pa::CacheDims c;
    pa_status_t s = check_cache(dtype, num_blocks, num_kv_heads, head_dim, &c);
    if (s != PA_OK)
        return s;
    REQUIRE(num_seqs >= 0, "num_seqs %d < 0", num_seqs);
    REQUIRE(total_q >= 0, "total_q %d < 0", total_q);
    REQUIRE(max_q_len >= 0, "max_q_len %d < 0", max_q_len);
    if (tree)
        REQUIRE(max_q_len <= 64, "max_q_len %d > 64: a tree mask covers at most 64 rows", max_q_len);
    if (fp8)
        REQUIRE(good_scale(k_scale) && good_scale(v_scale),
                "k_scale %g / v_scale %g is not a finite positive number", (double)k_scale,
                (double)v_scale);
    REQUIRE(num_q_heads > 0 && num_q_heads % num_kv_heads == 0,
            "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
            num_kv_heads);
    REQUIRE(max_blocks_per_seq >= 0, "max_blocks_per_seq %d < 0", max_blocks_per_seq);
    REQUIRE(scale > 0.0f && scale < 3.0e38f, "scale %g is not a finite positive number", (double)scale);
    if (!pa::prefill_supported(head_dim, num_q_heads / num_kv_heads))
        return fail(PA_ERR_UNSUPPORTED, "no prefill kernel for head_dim %d, group %d", head_dim,
                    num_q_heads / num_kv_heads);
    if (num_seqs == 0 || total_q == 0)
        return ok();
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(query, "query");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    REQUIRE(block_tables != nullptr, "block_tables is NULL");
    REQUIRE(seq_lens != nullptr, "seq_lens is NULL");
    REQUIRE(cu_q_lens != nullptr, "cu_q_lens is NULL");
    if (tree) {
        REQUIRE(tree_mask != nullptr, "tree_mask is NULL");
        REQUIRE(((uintptr_t)tree_mask & 7) == 0, "tree_mask is not 8-byte aligned");
    }
    pa::PrefillLaunch p;
    p.c = c;
    p.out = out;
    p.query = query;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.max_blocks = max_blocks_per_seq;
    p.seq_lens = seq_lens;
    p.cu_q_lens = cu_q_lens;
    p.num_seqs = num_seqs;
    p.total_q = total_q;
    p.max_q_len = max_q_len;
    p.num_q_heads = num_q_heads;
    p.scale = scale;
    p.tree_mask = tree ? tree_mask : nullptr;
    p.c.fp8 = fp8;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    if (fp8 && workspace != nullptr) {
        REQUIRE(max_blocks_per_seq > 0, "max_blocks_per_seq %d: nothing to widen",
                max_blocks_per_seq);
        REQUIRE((int64_t)num_seqs * max_blocks_per_seq <= 0x7fffffff,
                "num_seqs * max_blocks_per_seq %lld exceeds the widened pool's block ids",
                (long long)num_seqs * max_blocks_per_seq);
        REQUIRE(((uintptr_t)workspace & 255) == 0, "workspace is not 256-byte aligned");
        const size_t need = pa::prefill_widen_bytes(num_seqs, max_blocks_per_seq, num_kv_heads,
                                                    head_dim);
        if (workspace_bytes < need)
            return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                        need);
        p.widen_k16 = workspace;
        p.widen_v16 = (char *)workspace + need / 2;
    }
    return launched(pa::launch_prefill(p, (hipStream_t)stream),
                    tree ? "prefill_chunk_tree" : fp8 ? "prefill_chunk_fp8" : "prefill_chunk");
}

}  // namespace

extern "C" {

pa_status_t pa_prefill_chunk(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                             int32_t head_dim, void *out, const void *query,
                             const void *k_cache, const void *v_cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *seq_lens, const int32_t *cu_q_lens,
                             int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                             int32_t num_q_heads, float scale, void *stream)
{
    return prefill_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                        block_tables, max_blocks_per_seq, seq_lens, cu_q_lens, nullptr, false,
                        num_seqs, total_q, max_q_len, num_q_heads, scale, stream);
}

size_t pa_prefill_chunk_fp8_workspace_size(int32_t num_seqs, int32_t max_blocks_per_seq,
                                           int32_t num_kv_heads, int32_t head_dim)
{
    return pa::prefill_widen_bytes(num_seqs, max_blocks_per_seq, num_kv_heads, head_dim);
}

pa_status_t pa_prefill_chunk_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                 int32_t head_dim, void *out, const void *query,
                                 const void *k_cache, const void *v_cache,
                                 const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *seq_lens, const int32_t *cu_q_lens,
                                 int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                 int32_t num_q_heads, float scale, float k_scale, float v_scale,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    return prefill_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                        block_tables, max_blocks_per_seq, seq_lens, cu_q_lens, nullptr, false,
                        num_seqs, total_q, max_q_len, num_q_heads, scale, stream, true, k_scale,
                        v_scale, workspace, workspace_bytes);
}

pa_status_t pa_prefill_chunk_tree(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                  int32_t head_dim, void *out, const void *query,
                                  const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *seq_lens, const int32_t *cu_q_lens,
                                  const uint64_t *tree_mask, int32_t num_seqs, int32_t total_q,
                                  int32_t max_q_len, int32_t num_q_heads, float scale,
                                  void *stream)
{
    return prefill_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                        block_tables, max_blocks_per_seq, seq_lens, cu_q_lens, tree_mask, true,
                        num_seqs, total_q, max_q_len, num_q_heads, scale, stream);
}

}  // extern "C"

extern "C" {

size_t pa_decode_multi_workspace_size(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_seq_len,
                                      int32_t partition_size)
{
    if (parts_of(max_seq_len, partition_size) == 0)
        return 0;
    return pa::decode_multi_workspace_used(num_seqs, max_q_len, num_q_heads, head_dim,
                                           max_seq_len, partition_size);
}

}  // extern "C"

namespace {

pa_status_t multi_call(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                       int32_t head_dim, void *out, const void *query, const void *k_cache,
                       const void *v_cache, const int32_t *block_tables,
                       int32_t max_blocks_per_seq, const int32_t *seq_lens,
                       const int32_t *cu_q_lens, const uint64_t *tree_mask, int32_t num_seqs,
                       int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                       int32_t num_q_heads, float scale, int32_t partition_size, void *workspace,
                       size_t workspace_bytes, void *stream, bool fp8, float k_scale,
                       float v_scale)
{
    pa::CacheDims c;
    pa_status_t s = check_cache(dtype, num_blocks, num_kv_heads, head_dim, &c);
    if (s != PA_OK)
        return s;
    REQUIRE(num_seqs >= 0, "num_seqs %d < 0", num_seqs);
    REQUIRE(total_q >= 0, "total_q %d < 0", total_q);
    REQUIRE(max_q_len >= 1 && max_q_len <= pa::kMultiMaxRows, "max_q_len %d is outside [1, %d]",
            max_q_len, pa::kMultiMaxRows);
    REQUIRE(num_q_heads > 0 && num_q_heads % num_kv_heads == 0,
            "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
            num_kv_heads);
    REQUIRE(max_blocks_per_seq >= 0, "max_blocks_per_seq %d < 0", max_blocks_per_seq);
    REQUIRE(max_seq_len >= 0 && (int64_t)max_seq_len <= (int64_t)PA_BLOCK_SIZE * max_blocks_per_seq,
            "max_seq_len %d is outside [0, 16 * max_blocks_per_seq = %lld]", max_seq_len,
            (long long)PA_BLOCK_SIZE * max_blocks_per_seq);
    REQUIRE(partition_size >= 0 && partition_size % PA_BLOCK_SIZE == 0 && partition_size <= 1024,
            "partition_size %d is not 0 or a multiple of 16 up to 1024", partition_size);
    REQUIRE(scale > 0.0f && scale < 3.0e38f, "scale %g is not a finite positive number", (double)scale);
    if (fp8)
        REQUIRE(good_scale(k_scale) && good_scale(v_scale),
                "k_scale %g / v_scale %g is not a finite positive number", (double)k_scale,
                (double)v_scale);
    // row indices (total_q rows, or sequence x max_q_len rows, times the heads) stay in int32
    REQUIRE((int64_t)total_q * num_q_heads <= 0x7fffffff &&
                (int64_t)num_seqs * max_q_len * num_q_heads <= 0x7fffffff,
            "%d query rows x %d heads exceed the row index range", total_q, num_q_heads);
    if (!pa::decode_supported(head_dim, num_q_heads / num_kv_heads))
        return fail(PA_ERR_UNSUPPORTED, "no decode kernel for head_dim %d, group %d", head_dim,
                    num_q_heads / num_kv_heads);
    if (num_seqs == 0 || total_q == 0)
        return ok();
    REQUIRE_PTR(out, "out");
    REQUIRE_PTR(query, "query");
    REQUIRE_PTR(k_cache, "k_cache");
    REQUIRE_PTR(v_cache, "v_cache");
    REQUIRE(block_tables != nullptr, "block_tables is NULL");
    REQUIRE(seq_lens != nullptr, "seq_lens is NULL");
    REQUIRE(cu_q_lens != nullptr, "cu_q_lens is NULL");
    if (tree_mask != nullptr)
        REQUIRE(((uintptr_t)tree_mask & 7) == 0, "tree_mask is not 8-byte aligned");
    const size_t need = pa_decode_multi_workspace_size(num_seqs, max_q_len, num_q_heads, head_dim,
                                                       max_seq_len, partition_size);
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                        need);
        REQUIRE(aligned16(workspace), "workspace is not 16-byte aligned");
    }
    pa::DecodeLaunch d;
    d.c = c;
    d.out = out;
    d.query = query;
    d.k_cache = k_cache;
    d.v_cache = v_cache;
    d.block_tables = block_tables;
    d.max_blocks = max_blocks_per_seq;
    d.seq_lens = seq_lens;
    d.num_seqs = num_seqs;
    d.max_seq_len = max_seq_len;
    d.num_q_heads = num_q_heads;
    d.scale = scale;
    d.partition_size = partition_size;
    d.max_parts = parts_of(max_seq_len, partition_size);
    d.seq_starts = nullptr;
    d.group_starts = nullptr;
    d.num_groups = 0;
    d.max_group_size = 0;
    d.max_prefix_len = 0;
    d.workspace = need > 0 ? workspace : nullptr;
    d.fp8 = fp8;
    d.c.fp8 = fp8;
    d.k_scale = k_scale;
    d.v_scale = v_scale;
    d.cu_q_lens = cu_q_lens;
    d.tree_mask = tree_mask;
    d.max_q_len = max_q_len;
    d.total_q = total_q;
    return launched(pa::launch_decode_multi(d, (hipStream_t)stream),
                    fp8 ? "decode_multi_fp8" : "decode_multi");
}

}  // namespace

extern "C" {

pa_status_t pa_decode_multi(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                            int32_t head_dim, void *out, const void *query, const void *k_cache,
                            const void *v_cache, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens,
                            const int32_t *cu_q_lens, const uint64_t *tree_mask, int32_t num_seqs,
                            int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                            int32_t num_q_heads, float scale, int32_t partition_size,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    return multi_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                      block_tables, max_blocks_per_seq, seq_lens, cu_q_lens, tree_mask, num_seqs,
                      total_q, max_q_len, max_seq_len, num_q_heads, scale, partition_size,
                      workspace, workspace_bytes, stream, false, 1.0f, 1.0f);
}

pa_status_t pa_decode_multi_fp8(pa_dtype_t dtype, int32_t num_blocks, int32_t num_kv_heads,
                                int32_t head_dim, void *out, const void *query,
                                const void *k_cache, const void *v_cache,
                                const int32_t *block_tables, int32_t max_blocks_per_seq,
                                const int32_t *seq_lens, const int32_t *cu_q_lens,
                                const uint64_t *tree_mask, int32_t num_seqs, int32_t total_q,
                                int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                                float scale, float k_scale, float v_scale,
                                int32_t partition_size, void *workspace, size_t workspace_bytes,
                                void *stream)
{
    return multi_call(dtype, num_blocks, num_kv_heads, head_dim, out, query, k_cache, v_cache,
                      block_tables, max_blocks_per_seq, seq_lens, cu_q_lens, tree_mask, num_seqs,
                      total_q, max_q_len, max_seq_len, num_q_heads, scale, partition_size,
                      workspace, workspace_bytes, stream, true, k_scale, v_scale);
}

}  // extern "C"
