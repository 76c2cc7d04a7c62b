// pa_shapes.cpp -- host-side shape logic shared by the C ABI's checks and the kernel launchers:
// which head dimensions and groups have kernels, and how many bytes of partial results a split
// decode keeps. No device code; it builds with any C++17 compiler.
#include "pa_internal.h"

namespace pa {

bool decode_supported(int32_t head_dim, int32_t group)
{
    return (head_dim == 64 || head_dim == 128) && group >= 1;
}

bool prefill_supported(int32_t head_dim, int32_t group)
{
    return (head_dim == 64 || head_dim == 128) && group >= 1;
}

size_t decode_workspace_used(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_seq_len, int32_t partition_size)
{
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        partition_size <= 0 || max_seq_len <= partition_size)
        return 0;  // unsplit: no partial results
    const int parts = (max_seq_len + partition_size - 1) / partition_size;
    // groups of 1-2 query heads: one part per slot (vector-ALU kernel); larger groups: the MFMA
    // kernel's workgroups merge kDecodeMfmaWaves consecutive parts into one slot
    const int wg_parts = num_q_heads / num_kv_heads <= 2 ? 1 : kDecodeMfmaWaves;
    const size_t slots = (size_t)(parts + wg_parts - 1) / wg_parts;
    return (size_t)num_seqs * num_q_heads * slots * (head_dim + 2) * sizeof(float);
}

size_t decode_multi_workspace_used(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                   int32_t head_dim, int32_t max_seq_len, int32_t partition_size)
{
    if (num_seqs <= 0 || max_q_len <= 0 || num_q_heads <= 0 || head_dim <= 0 ||
        partition_size <= 0 || max_seq_len <= 0)
        return 0;  // unsplit: no partial results
    const int parts = (max_seq_len + partition_size - 1) / partition_size;
    const size_t slots = (size_t)(parts + kDecodeMfmaWaves - 1) / kDecodeMfmaWaves;
    return (size_t)num_seqs * max_q_len * num_q_heads * slots * (head_dim + 2) * sizeof(float);
}

size_t prefill_widen_bytes(int32_t num_seqs, int32_t max_blocks, int32_t num_kv_heads,
                           int32_t head_dim)
{
    if (num_seqs <= 0 || max_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return 0;
    // K and V, 16-bit elements, blocks of 16 rows: one region per cache, 256-byte aligned
    const size_t region = (size_t)num_seqs * max_blocks * num_kv_heads * 16 * head_dim * 2;
    return 2 * ((region + 255) & ~(size_t)255);
}

}  // namespace pa
