// reshape_and_cache.hip -- scatter the new tokens' K and V rows into their cache slots.
//
// Lecture 32 "LLM 在线推理两阶段" §3.1: each decode step appends its new k_t, v_t to the cache;
// openeuler.csdn.net "高并发 AI 服务的内存瓶颈", Block Table 数据结构: the slot of a position is
// physical_block * 16 + offset. A bit copy: every 16-byte piece of a token's [H_kv][D] key/value
// row goes to the same piece of its (block, kv head, offset) row in the cache.
//
// Layout: key/value [T][H_kv][D]; cache [num_blocks][H_kv][16][D]. One thread moves 16 bytes of K
// and 16 bytes of V; consecutive threads read consecutive input bytes (coalesced) and write whole
// 16-byte pieces of a D-element cache row (a 128/256-byte run per head).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint4 *__restrict__ k_cache,
    uint4 *__restrict__ v_cache, const int32_t *__restrict__ slot_mapping, int32_t num_tokens,
    int32_t num_blocks, int32_t num_kv_heads, int32_t vec_per_row /* D / 8 */)
{
    const int32_t vec_per_token = num_kv_heads * vec_per_row;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)num_tokens * vec_per_token)
        return;
    const int32_t t = (int32_t)(i / vec_per_token);
    const int32_t v = (int32_t)(i % vec_per_token);
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * kBlock)  // negative: padding; beyond the pool: skipped
        return;
    const int32_t blk = slot / kBlock, off = slot % kBlock;
    const int32_t head = v / vec_per_row, piece = v % vec_per_row;
    const int64_t dst = (((int64_t)blk * num_kv_heads + head) * kBlock + off) * vec_per_row + piece;
    k_cache[dst] = key[i];
    v_cache[dst] = value[i];
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheDims &c, const void *key, const void *value,
                                    void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                    int32_t num_tokens, hipStream_t stream)
{
    const int32_t vec_per_row = c.head_dim / 8;
    const int64_t total = (int64_t)num_tokens * c.num_kv_heads * vec_per_row;
    if (total == 0)
        return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4 *)key, (const uint4 *)value, (uint4 *)k_cache,
                       (uint4 *)v_cache, slot_mapping, num_tokens, c.num_blocks, c.num_kv_heads,
                       vec_per_row);
    return hipGetLastError();
}

}  // namespace pa
