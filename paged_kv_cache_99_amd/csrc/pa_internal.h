// pa_internal.h -- launch-side interface between the C ABI (pa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Set the calling thread's pa_last_error() message and return s (pa_api.cpp).
pa_status_t fail(pa_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return PA_OK.
pa_status_t ok();

struct CacheDims {
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t head_dim;
    bool bf16;          // 16-bit element type of queries, keys, values and outputs
    bool fp8 = false;   // the caches hold E4M3 codes (one byte per element)
};

// reshape_and_cache.hip
hipError_t launch_reshape_and_cache(const CacheDims &c, const void *key, const void *value,
                                    void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                    int32_t num_tokens, hipStream_t stream);
// E4M3 caches: the code of x / k_scale (keys) or x / v_scale (values) goes to the slot.
hipError_t launch_reshape_and_cache_fp8(const CacheDims &c, const void *key, const void *value,
                                        void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                        int32_t num_tokens, float k_scale, float v_scale,
                                        hipStream_t stream);

// copy_blocks.hip
hipError_t launch_copy_blocks(const CacheDims &c, void *k_cache, void *v_cache,
                              const int32_t *block_mapping, int32_t num_pairs, hipStream_t stream);

// decode.hip
struct DecodeLaunch {
    CacheDims c;
    void *out;
    const void *query;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks;
    const int32_t *seq_lens;
    int32_t num_seqs;
    int32_t max_seq_len;
    int32_t num_q_heads;
    float scale;
    int32_t partition_size;  // 0 = unsplit
    float *ws_acc;           // [num_seqs][num_q_heads][max_parts][head_dim]
    float *ws_ml;            // [num_seqs][num_q_heads][slots][2]
    int32_t max_parts;       // own parts per sequence (0 = unsplit)
    // shared-prefix (cascade) decode; group_starts == nullptr for a plain decode
    const int32_t *seq_starts;    // [num_seqs] shared-prefix length of each sequence
    const int32_t *group_starts;  // [num_groups + 1]
    int32_t num_groups;
    int32_t max_group_size;
    int32_t max_prefix_len;
    // E4M3 caches (c.fp8): element = code value * k_scale / v_scale
    bool fp8 = false;
    float k_scale = 1.0f;
    float v_scale = 1.0f;
};
// Group sizes with a dedicated kernel; any other group size runs as several of these.
bool decode_supported(int32_t head_dim, int32_t group);
hipError_t launch_decode(const DecodeLaunch &d, hipStream_t stream);

// prefill.hip
struct PrefillLaunch {
    CacheDims c;
    void *out;
    const void *query;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    int32_t max_blocks;
    const int32_t *seq_lens;
    const int32_t *cu_q_lens;
    const uint64_t *tree_mask = nullptr;  // drafted-token trees: one mask per query row
    int32_t num_seqs;
    int32_t total_q;
    int32_t max_q_len;
    int32_t num_q_heads;
    float scale;
    // E4M3 caches (c.fp8): element = code value * k_scale / v_scale; query/out of dtype c.bf16
    float k_scale = 1.0f;
    float v_scale = 1.0f;
};
bool prefill_supported(int32_t head_dim, int32_t group);
hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream);

}  // namespace pa
