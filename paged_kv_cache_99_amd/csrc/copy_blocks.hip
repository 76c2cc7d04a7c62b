// copy_blocks.hip -- copy-on-write of shared physical blocks.
//
// openeuler.csdn.net "高并发 AI 服务的内存瓶颈", section 机制 2 写时复制: sequences that share a
// prompt's blocks (reference-counted) get a private copy of a block where they diverge. The whole
// block -- 16 slots x all kv heads, filled or not -- is copied in both caches, bit for bit (16-bit
// or E4M3 elements alike).
//
// Grid: x = pair, y = 16 KiB piece of the block, z = cache (0: K, 1: V). Each thread moves four
// 16-byte vectors, issuing all four loads before the stores. The stores are nontemporal: a decode
// that follows in the same step then does not pay for their write-back amid its reads (224
// copy-on-write pairs of 32-head blocks, 57 MB, cost a following decode ~35 us when written back
// later).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int kVecPerWg = kThreads * kVecPerThread;  // 16 KiB per workgroup

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache,
    const int32_t *__restrict__ block_mapping, int32_t num_blocks, int32_t vec_per_block)
{
    const int32_t src = block_mapping[2 * blockIdx.x];
    const int32_t dst = block_mapping[2 * blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
        return;  // a pair outside the pool is skipped
    uint4 *cache = blockIdx.z == 0 ? k_cache : v_cache;
    const uint4 *from = cache + (int64_t)src * vec_per_block;
    uint4 *to = cache + (int64_t)dst * vec_per_block;
    const int32_t first = blockIdx.y * kVecPerWg + threadIdx.x;
    uint4 r[kVecPerThread];
#pragma unroll
    for (int k = 0; k < kVecPerThread; ++k) {
        const int32_t i = first + k * kThreads;
        if (i < vec_per_block)
            r[k] = from[i];
    }
#pragma unroll
    for (int k = 0; k < kVecPerThread; ++k) {
        const int32_t i = first + k * kThreads;
        if (i < vec_per_block)
            store_nt(&to[i], r[k]);
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CacheDims &c, void *k_cache, void *v_cache,
                              const int32_t *block_mapping, int32_t num_pairs, hipStream_t stream)
{
    if (num_pairs == 0)
        return hipSuccess;
    const int32_t vec_per_block = c.num_kv_heads * kBlock * c.head_dim * (c.fp8 ? 1 : 2) / 16;
    const int32_t pieces = (vec_per_block + kVecPerWg - 1) / kVecPerWg;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, pieces, 2), dim3(kThreads), 0, stream,
                       (uint4 *)k_cache, (uint4 *)v_cache, block_mapping, c.num_blocks,
                       vec_per_block);
    return hipGetLastError();
}

}  // namespace pa
