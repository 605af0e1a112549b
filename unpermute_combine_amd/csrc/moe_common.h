// Internal helpers shared by the gfx950 kernels of libmoe_dispatch.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dispatch.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------- bf16 <-> float32
// bf16 is the upper half of an IEEE float32; widening is a shift, narrowing rounds to nearest
// with ties to even (NaN kept quiet with its sign; element-wise paths).
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

// Two values rounded to bf16 by gfx950's conversion instruction (v_cvt_pk_bf16_f32: nearest, ties
// to even; bit for bit f32_to_bf16_bits on finite values, ties, subnormals and overflow), lo in the
// low half. One instruction per pair instead of ~6 integer operations per value: measured with
// caches flushed, the weighted scatter of the combine's backward at T16384 H7168 K8 went 408 ->
// ~365 us (it was ALU-bound) and the batched combine 344 -> 341 us.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
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

__device__ __forceinline__ void st16_stream(void *p, const u32x4 &v)
{
    uint32_t *q = reinterpret_cast<uint32_t *>(p);
    __builtin_nontemporal_store(v.x, q + 0);
    __builtin_nontemporal_store(v.y, q + 1);
    __builtin_nontemporal_store(v.z, q + 2);
    __builtin_nontemporal_store(v.w, q + 3);
}

// ---------------------------------------------------------------- buffer resources
// A buffer resource (base address + size in bytes) gives loads and stores explicit gfx950
// cache-policy bits and a hardware bounds check (accesses past the size read 0 / are dropped).
// Policy bits of the aux operand: 1 = sc0, 2 = nt (streaming), 16 = sc1.
//   kPolicyStreamStore = sc1|nt: agent-scope streaming store, written through the per-XCD L2
//                        (measured: the expert-major permute writes at ~6.0 TB/s instead of ~5.4);
//   kPolicyStreamLoad  = sc0|nt: streaming load of data read exactly once;
//   kPolicyNontemporal = nt: streaming store at the default scope (the combine's outputs);
//   kPolicyDeviceStore = sc1: agent-scope store with the normal cache policy (the pre-combine's
//                        partials, which it writes 4-10% faster than with nt or sc1|nt).
constexpr int kPolicyStreamLoad = 1 | 2;
constexpr int kPolicyStreamStore = 16 | 2;
constexpr int kPolicyNontemporal = 2;
constexpr int kPolicyDeviceStore = 16;
constexpr int kRsrcWord3 = 0x00020000;  // dword 3 of the resource: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

template <int AUX>
__device__ __forceinline__ u32x4 ld16_buf(__amdgpu_buffer_rsrc_t r, uint32_t offset)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(offset), 0, AUX);
    return u32x4{static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                 static_cast<uint32_t>(v[3])};
}

template <int AUX>
__device__ __forceinline__ void st16_buf(__amdgpu_buffer_rsrc_t r, uint32_t offset, const u32x4 &q)
{
    __attribute__((ext_vector_type(4))) unsigned int v = {q.x, q.y, q.z, q.w};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(offset), 0, AUX);
}

__device__ __forceinline__ uint64_t lanemask_lt()
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Workgroups are dispatched to the 8 XCDs round-robin (block b to XCD b % 8). This renumbers the
// blocks so that each XCD takes one contiguous range of logical blocks (XCD x the x-th eighth,
// the first nb % 8 XCDs one block more), a bijection on [0, nb).
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t b, uint32_t nb)
{
    const uint32_t per = nb / kXcds, extra = nb % kXcds;
    const uint32_t x = b % kXcds, i = b / kXcds;
    return x < extra ? x * (per + 1) + i : extra * (per + 1) + (x - extra) * per + i;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline moe_status launch_status()
{
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The source-major row scatter of moe_permute_scatter for rows of nvec 16-byte vectors (permute.hip):
// dst[dst_of[t*J + j]] = src[t]; rows i with src_row[i] outside [0, src_rows) other than
// MOE_ROW_UNUSED become zero rows (src_row may be NULL). With `scaled`, the rows are bf16 and
// destination j receives scale[t*J + j] * src[t] (float32 products rounded to bf16; scale NULL:
// unit weights). Launches on `stream`; sizes are the caller's to check.
moe_status launch_scatter_vec16(const char *src, int64_t src_rows, int64_t nvec, const int32_t *dst_of, int J,
                                const int32_t *src_row, int64_t N, char *dst, bool scaled, const float *scale,
                                hipStream_t stream);

// moe_build_index's rank pass over tile counts already in `workspace` (tiles of tile_tokens whole
// tokens, the last one partial; per tile a row of round4(E) expert counts followed, with groups,
// by round4(E / group_size) counts of each token's first slot per group; at most 256 tiles, rows
// 16-byte aligned). launch = false checks the arguments only. Same outputs as moe_build_index.
moe_status build_index_from_tile_counts(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K, int32_t E,
                                        int32_t capacity, int32_t group_size, int32_t alignment, const moe_index *out,
                                        void *workspace, size_t workspace_bytes, int32_t tile_tokens, bool launch,
                                        hipStream_t stream);
// True when moe_build_index counts the tiles in a launch of its own for these sizes.
bool build_index_counts_tiles(int64_t T, int32_t K);

}  // namespace moe
