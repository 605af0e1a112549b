// Internal helpers shared by the gfx950 kernels of libmoe_dispatch.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dispatch.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------- bf16 <-> float32
// bf16 is the upper half of an IEEE float32; widening is a shift, narrowing rounds to nearest
// with ties to even (NaN kept quiet with its sign).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x0040u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 16-byte vector used for every row access (global_load/store_dwordx4).
struct alignas(16) u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 ld16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void st16(void *p, const u32x4 &v)
{
    *reinterpret_cast<u32x4 *>(p) = v;
}

__device__ __forceinline__ u32x4 ld16_stream(const void *p)
{
    u32x4 v;
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
    v.x = __builtin_nontemporal_load(q + 0);
    v.y = __builtin_nontemporal_load(q + 1);
    v.z = __builtin_nontemporal_load(q + 2);
    v.w = __builtin_nontemporal_load(q + 3);
    return v;
}

__device__ __forceinline__ void st16_stream(void *p, const u32x4 &v)
{
    uint32_t *q = reinterpret_cast<uint32_t *>(p);
    __builtin_nontemporal_store(v.x, q + 0);
    __builtin_nontemporal_store(v.y, q + 1);
    __builtin_nontemporal_store(v.z, q + 2);
    __builtin_nontemporal_store(v.w, q + 3);
}

__device__ __forceinline__ uint64_t lanemask_lt()
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline moe_status launch_status()
{
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe
