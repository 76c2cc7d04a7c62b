// reshape_and_cache.hip -- scatter the new tokens' K and V rows into their cache slots.
//
// Lecture 32 "LLM 在线推理两阶段" §3.1: each decode step appends its new k_t, v_t to the cache;
// openeuler.csdn.net "高并发 AI 服务的内存瓶颈", Block Table 数据结构: the slot of a position is
// physical_block * 16 + offset. A bit copy: every 16-byte piece of a token's [H_kv][D] key/value
// row goes to the same piece of its (block, kv head, offset) row in the cache.
//
// Layout: key/value [T][H_kv][D]; cache [num_blocks][H_kv][16][D]. One thread moves 16 bytes of K
// and 16 bytes of V; consecutive threads read consecutive input bytes (coalesced) and write whole
// 16-byte pieces of a D-element cache row (a 128/256-byte run per head), with nontemporal stores
// (the attention kernels of the step stream their reads while ordinary stores would still be
// waiting in the caches to be written back).
//
// E4M3 caches (lecture 34 "vLLM 生产级系统架构全景剖析" §4.4: one byte per key and value element):
// a thread reads 16 elements (32 bytes) of K and of V and writes their 16 codes. The code of x is
// the E4M3 value nearest to x / scale -- the quotient rounded to float32, ties to the even code,
// magnitudes of 448 and beyond saturated to 448 -- and a NaN element gets the NaN code 0x7F with its
// sign.
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
    store_nt(&k_cache[dst], key[i]);
    store_nt(&v_cache[dst], value[i]);
}

// Codes of the four 16-bit elements of (w0, w1), element j in byte j.
template <bool BF>
__device__ __forceinline__ uint32_t quantize4(uint32_t w0, uint32_t w1, float scale)
{
    const float x[4] = {lo_f32<BF>(w0), hi_f32<BF>(w0), lo_f32<BF>(w1), hi_f32<BF>(w1)};
    float q[4];
    uint32_t nan_mask = 0, nan_codes = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        q[j] = fminf(fmaxf(x[j] / scale, -448.0f), 448.0f);  // IEEE division, then saturate
        if (x[j] != x[j]) {
            nan_mask |= 0xFFu << (8 * j);
            nan_codes |= (0x7Fu | (__float_as_uint(x[j]) >> 31 << 7)) << (8 * j);
        }
    }
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);  // bytes 0, 1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);            // bytes 2, 3
    return (w & ~nan_mask) | nan_codes;
}

template <bool BF>
__device__ __forceinline__ uint4 quantize16(const uint4 &a, const uint4 &b, float scale)
{
    return make_uint4(quantize4<BF>(a.x, a.y, scale), quantize4<BF>(a.z, a.w, scale),
                      quantize4<BF>(b.x, b.y, scale), quantize4<BF>(b.z, b.w, scale));
}

template <bool BF>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint4 *__restrict__ key, const uint4 *__restrict__ value, uint4 *__restrict__ k_cache,
    uint4 *__restrict__ v_cache, const int32_t *__restrict__ slot_mapping, int32_t num_tokens,
    int32_t num_blocks, int32_t num_kv_heads, int32_t pieces_per_row /* D / 16 */, float k_scale,
    float v_scale)
{
    const int32_t pieces_per_token = num_kv_heads * pieces_per_row;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-element piece
    if (i >= (int64_t)num_tokens * pieces_per_token)
        return;
    const int32_t t = (int32_t)(i / pieces_per_token);
    const int32_t v = (int32_t)(i % pieces_per_token);
    const int32_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * kBlock)  // negative: padding; beyond the pool: skipped
        return;
    const int32_t blk = slot / kBlock, off = slot % kBlock;
    const int32_t head = v / pieces_per_row, piece = v % pieces_per_row;
    const int64_t dst = (((int64_t)blk * num_kv_heads + head) * kBlock + off) * pieces_per_row + piece;
    store_nt(&k_cache[dst], quantize16<BF>(key[2 * i], key[2 * i + 1], k_scale));
    store_nt(&v_cache[dst], quantize16<BF>(value[2 * i], value[2 * i + 1], v_scale));
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

hipError_t launch_reshape_and_cache_fp8(const CacheDims &c, const void *key, const void *value,
                                        void *k_cache, void *v_cache, const int32_t *slot_mapping,
                                        int32_t num_tokens, float k_scale, float v_scale,
                                        hipStream_t stream)
{
    const int32_t pieces_per_row = c.head_dim / 16;
    const int64_t total = (int64_t)num_tokens * c.num_kv_heads * pieces_per_row;
    if (total == 0)
        return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    auto kern = c.bf16 ? reshape_and_cache_fp8_kernel<true> : reshape_and_cache_fp8_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(threads), 0, stream, (const uint4 *)key,
                       (const uint4 *)value, (uint4 *)k_cache, (uint4 *)v_cache, slot_mapping,
                       num_tokens, c.num_blocks, c.num_kv_heads, pieces_per_row, k_scale, v_scale);
    return hipGetLastError();
}

}  // namespace pa
