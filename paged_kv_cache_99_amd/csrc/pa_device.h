// pa_device.h -- device-side helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Marks a lambda always inlined (arrays it takes by reference then stay in registers).
#define PA_INLINE __attribute__((always_inline))

constexpr int kBlock = 16;  // tokens per physical block
constexpr int kWave = 64;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ 16-bit words <-> float32
template <bool BF>
__device__ __forceinline__ float lo_f32(uint32_t w)  // low 16-bit element of a 32-bit word
{
    if constexpr (BF) {
        return __uint_as_float(w << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
}

template <bool BF>
__device__ __forceinline__ float hi_f32(uint32_t w)  // high 16-bit element
{
    if constexpr (BF) {
        return __uint_as_float(w & 0xffff0000u);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
}

// Round float32 values to the 16-bit type, nearest even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 on
// gfx950; NaN stays NaN).
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (BF) {
        const bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        const f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <bool BF>
__device__ __forceinline__ uint32_t to_word(float x)
{
    if constexpr (BF) {
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
    } else {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
    }
}

// c + a.lo*b.lo + a.hi*b.hi in float32 (v_dot2_f32_f16 / v_dot2_f32_bf16).
template <bool BF>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    if constexpr (BF) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                               __builtin_bit_cast(bf16x2, b), c, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                      c, false);
    }
}

// Dot product of two runs of 8 16-bit elements held in 16-byte vectors.
template <bool BF>
__device__ __forceinline__ float dot8(const uint4 &a, const uint4 &b)
{
    float s = dot2<BF>(a.x, b.x, 0.0f);
    s = dot2<BF>(a.y, b.y, s);
    s = dot2<BF>(a.z, b.z, s);
    return dot2<BF>(a.w, b.w, s);
}

// ------------------------------------------------------------------ FP8 (E4M3) cache elements
// gfx950's FP8 conversions read and write the OCP E4M3 format (bias 7, no infinities, largest 448).
// Every E4M3 value is exactly an f16, a bf16 and a float32 value.

// Codes in bytes 0,1 (HI = false) or 2,3 (HI = true) of w as two 16-bit elements, low half first
// (v_cvt_scalef32_pk_{f16,bf16}_fp8 with scale 1: exact).
template <bool BF, bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_pk16(uint32_t w)
{
    if constexpr (BF)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Dot product of 16 16-bit query elements (q[0]: elements 0..7, q[1]: 8..15) with the 16 E4M3
// codes of k (byte j = element j).
template <bool BF>
__device__ __forceinline__ float dot16_e4m3(const uint4 (&q)[2], const uint4 &k)
{
    const uint4 a = make_uint4(e4m3x2_to_pk16<BF, false>(k.x), e4m3x2_to_pk16<BF, true>(k.x),
                               e4m3x2_to_pk16<BF, false>(k.y), e4m3x2_to_pk16<BF, true>(k.y));
    const uint4 b = make_uint4(e4m3x2_to_pk16<BF, false>(k.z), e4m3x2_to_pk16<BF, true>(k.z),
                               e4m3x2_to_pk16<BF, false>(k.w), e4m3x2_to_pk16<BF, true>(k.w));
    return dot8<BF>(q[0], a) + dot8<BF>(q[1], b);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// The four codes of w (byte j = element j) as float32 (v_cvt_pk_f32_fp8: exact).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float (&f)[4])
{
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
}

// ------------------------------------------------------------------ cross-lane reductions (DPP)
// DPP controls of GFX9: quad_perm(1,0,3,2) swaps neighbours, quad_perm(2,3,0,1) swaps pairs,
// row_half_mirror reverses each 8-lane half row, row_mirror reverses each 16-lane row.
__device__ __forceinline__ float dpp_f(float v, int ctrl_id)
{
    int x = __float_as_int(v);
    switch (ctrl_id) {
    case 0: x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true); break;
    case 1: x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); break;
    case 2: x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true); break;
    default: x = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true); break;
    }
    return __int_as_float(x);
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of a group gets the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    v += dpp_f(v, 0);
    v += dpp_f(v, 1);
    if constexpr (N >= 8)
        v += dpp_f(v, 2);
    if constexpr (N == 16)
        v += dpp_f(v, 3);
    return v;
}

__device__ __forceinline__ float xor_shfl(float v, int mask)
{
    return __shfl_xor(v, mask, kWave);
}

// Lanes l and l ^ 32 combined (v_permlane32_swap_b32 with both operands = v gives, at every lane,
// v of lanes l % 32 and 32 + l % 32 -- the lane and its partner, in lane order, so both partners
// compute the same result bit for bit).
__device__ __forceinline__ float pair_max(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v)
{
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, xor_shfl(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
    for (int m = 32; m >= 1; m >>= 1)
        v += xor_shfl(v, m);
    return v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked nontemporal (global_load_dwordx4 ... nt): for data streamed once, such as
// the K/V tiles of a decode step; it measurably raises the sustained read rate of scattered
// 4 KiB tiles on gfx950.
__device__ __forceinline__ uint4 load_nt(const void *p)
{
    const u32x4 t = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(t[0], t[1], t[2], t[3]);
}

// 16-byte store marked nontemporal (global_store_dwordx4 ... nt), for cache writes that the next
// kernels of the step do not read back soon: the lines leave the caches with the writing kernel
// instead of being written back to HBM while a following HBM-bound kernel streams its reads.
__device__ __forceinline__ void store_nt(void *p, const uint4 &v)
{
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, (u32x4 *)p);
}

// 16-byte direct-to-LDS load (global_load_lds_dwordx4, scalar-base form): lane i reads the 16
// bytes at sbase + voff_i and writes them to LDS address lds + 16 * i; sbase and lds are
// wave-uniform. M0 carries the LDS address and needs one wait state (s_nop 0) before the load
// reads it. Issued from inline assembly so that the compiler does not model the LDS write: it then
// inserts no wait for it before LDS reads of other buffers. The caller orders it -- s_waitcnt
// vmcnt and a barrier -- before its data is read or its buffer reused.
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(const lds_u8 *)p;
}

// 16-byte LDS read at byte address addr (ds_read_b128).
__device__ __forceinline__ uint4 lds_read16(uint32_t addr)
{
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)addr;
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void dma16_to_lds(uint32_t voff, const void *sbase, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ float fast_exp2(float x)
{
    return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// ------------------------------------------------------------------ launch helpers
// Workgroups are dealt to the 8 XCDs round-robin (workgroup w runs on XCD w % 8). Renumbering so
// that consecutive logical ids share an XCD keeps neighbouring work units on one L2.
__device__ __forceinline__ int xcd_logical_id(int wg, int grid)
{
    const int per_xcd = grid >> 3;  // grid is a multiple of 8
    return (wg & 7) * per_xcd + (wg >> 3);
}

__host__ __device__ constexpr int round_up8(int n) { return (n + 7) & ~7; }

}  // namespace pa
