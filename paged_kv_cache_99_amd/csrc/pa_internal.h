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
    // fp32 scratch of the partial results, laid out by launch_decode: acc [slots][rows][head_dim]
    // then (m, l) [rows][slots][2], rows = num_seqs * num_q_heads; decode_workspace_used bytes
    void *workspace;
    int32_t max_parts;       // own parts per sequence (0 = unsplit)
    // shared-prefix (cascade) decode; group_starts == nullptr for a plain decode
    const int32_t *seq_starts;    // [num_seqs] shared-prefix length of each sequence
    const int32_t *group_starts;  // [num_groups + 1]
    int32_t num_groups;
    int32_t max_group_size;
    int32_t max_prefix_len;
    int32_t max_own_len = 0;      // bound on seq_lens - prefix lens (shared-prefix decode); 0: none
    // E4M3 caches (c.fp8): element = code value * k_scale / v_scale
    bool fp8 = false;
    float k_scale = 1.0f;
    float v_scale = 1.0f;
    // multi-token decode (launch_decode_multi): up to max_q_len query rows per sequence, laid out
    // [total_q][num_q_heads][head_dim] by cu_q_lens [num_seqs + 1]; tree_mask [total_q] or null
    const int32_t *cu_q_lens = nullptr;
    const uint64_t *tree_mask = nullptr;
    int32_t max_q_len = 0;
    int32_t total_q = 0;
};
// Host-side shape logic (pa_shapes.cpp) ------------------------------------------------------
// The MFMA decode (head groups of 3 or more) runs workgroups of this many waves, and in a split
// decode each workgroup merges that many consecutive parts into one workspace slot.
constexpr int kDecodeMfmaWaves = 4;
// Group sizes with a dedicated kernel; any other group size runs as several of these.
bool decode_supported(int32_t head_dim, int32_t group);
hipError_t launch_decode(const DecodeLaunch &d, hipStream_t stream);
// Multi-token decode: the MFMA decode kernel over (row, query head) columns, rows of up to
// kMultiMaxRows per sequence; the workspace holds (sequence, row, head) partial rows.
constexpr int kMultiMaxRows = 16;
hipError_t launch_decode_multi(const DecodeLaunch &d, hipStream_t stream);
// Bytes of workspace a split multi-token decode writes and reads: one fp32 partial (head_dim + 2
// floats) per (sequence, row < max_q_len, query head) and slot of kDecodeMfmaWaves parts.
size_t decode_multi_workspace_used(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                   int32_t head_dim, int32_t max_seq_len, int32_t partition_size);
// Bytes of workspace a plain (unshared) decode of these sizes writes and reads: one fp32 partial
// (head_dim + 2 floats) per (sequence, query head, slot). At most pa_decode_workspace_size.
size_t decode_workspace_used(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_seq_len, int32_t partition_size);
// The library's static decode scratch (kDecodeScratchBytes) on the device that runs `stream`
// (the current device for the null stream): its address there, looked up once per device.
constexpr size_t kDecodeScratchBytes = PA_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch(hipStream_t stream, void **ptr);

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
    // E4M3 caches with a workspace: the sequences' blocks are first widened to 16 bits into these
    // two regions (num_seqs * max_blocks blocks each), and the 16-bit kernel runs on them
    void *widen_k16 = nullptr;
    void *widen_v16 = nullptr;
};
size_t prefill_widen_bytes(int32_t num_seqs, int32_t max_blocks, int32_t num_kv_heads,
                           int32_t head_dim);  // pa_shapes.cpp: both regions
bool prefill_supported(int32_t head_dim, int32_t group);  // pa_shapes.cpp
hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream);

}  // namespace pa
