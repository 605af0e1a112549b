// FP8 dispatch: per-block E4M3 quantization of the hidden rows, alone or fused into the
// source-major permute.
//
// [Combine] §3 ("03 · Combine 与 forward / backward 对称性"): DeepEP's dispatch sends FP8 while
// the combine stays BF16; [Megatron] ("token dispatcher + fuse_a2a", the DeepEP dispatch call):
// x travels together with x_scales, num_scales scale groups per token along the hidden
// dimension. Each token's hidden vector is cut into blocks of `block` consecutive elements; per
// block amax = max |x|, scale = amax / 448 (1 when amax is 0), and every element becomes the
// E4M3 code of x / scale (both divisions IEEE float32), rounded to nearest even and saturated at
// 448 -- the largest finite E4M3 value -- so x ~ value(code) * scale.
//
// gfx950 design. The codes come from the conversion instruction (v_cvt_pk_fp8_f32, two values
// per instruction, round to nearest even): it gives the definition's code for every finite
// E4M3 value, every tie between neighbours and the float32 neighbours of every tie (tested
// against the oracle), and replaced a bit-level encoder of ~12 instructions per element (the
// fused dispatch at T8192 H7168 in 32 groups: 73.7 -> 52.9 us; drop-and-pad T8192 H4096:
// 81.8 -> 69.0 us; unchanged at T16384 H7168 K8, where the stores dominate). The fused dispatch
// runs like the bf16 source-major permute -- one wavefront per (source row, 1024-element slice),
// each lane holding 16 consecutive elements -- with the block's amax reduced over the block's
// lanes by xor shuffles, then 16 codes (16 bytes) per lane stored to every destination row:
// 1 KiB per wavefront instruction, half the bytes of the bf16 rows. Scales are one float32 per
// block and row. Measured at T16384 H7168 K8: 212 us per launch (5.7 TB/s) against 241 us with
// 8 elements (8-byte stores) per lane; the divisions of the definition stay (multiplying by a
// reciprocal would change codes).
#include "moe_common.h"

namespace moe {
namespace {

constexpr float kE4M3Max = 448.0f;
constexpr int kFp8Slice = 1024;       // elements of a source row per wavefront (16 per lane)
constexpr int kFp8Threads = 256;
constexpr int kFp8Waves = kFp8Threads / kWave;
// padding rows checked per zero wavefront: with 4 KiB rows (H4096, drop-and-pad, caches flushed)
// 70.7 us with 8 rows, 75.1 with 4, 77.9 with 2 -- about 32 KiB of zeros per wave, as for the
// 8 KiB bf16 rows of the plain scatter (4 rows per wave)
constexpr int kFp8ZeroRows = 8;

// Four E4M3 codes packed in element order (byte i = code of the i-th value) by the gfx950
// conversion instruction (two values per instruction, round to nearest even into the OCP E4M3
// format). For finite x, |x / scale| exceeds 448 by at most the division's rounding, which
// rounds back to 448: the saturation of the definition is never needed beyond that.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return static_cast<uint32_t>(w);
}

__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false)) & 0xffu;
}

__device__ __forceinline__ float load_x(const uint16_t *p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }
__device__ __forceinline__ float load_x(const float *p) { return *p; }

// 8 consecutive elements of a row (16-byte aligned): bf16 one 16-byte load, float32 two.
__device__ __forceinline__ void load8x(const uint16_t *p, float (&v)[8])
{
    const u32x4 q = ld16(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}

__device__ __forceinline__ void load8x(const float *p, float (&v)[8])
{
    const u32x4 a = ld16(p), b = ld16(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

__device__ __forceinline__ float block_scale(float amax) { return amax > 0.0f ? amax / kE4M3Max : 1.0f; }

// ---------------------------------------------------------------- quantize (any block)
// One wavefront per (token, block): a pass for the block's amax, a pass for the codes.
template <typename X>
__global__ __launch_bounds__(kFp8Threads) void quantize_fp8_kernel(const X *__restrict__ x, int64_t T, int64_t H,
                                                                   int64_t block, uint8_t *__restrict__ q,
                                                                   float *__restrict__ scales)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nb = H / block;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kFp8Waves +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    if (gw >= T * nb)
        return;
    const int64_t t = gw / nb, b = gw - t * nb;
    const X *row = x + t * H + b * block;
    float amax = 0.0f;
    for (int64_t i = lane; i < block; i += kWave)
        amax = fmaxf(amax, fabsf(load_x(row + i)));
    for (int off = kWave / 2; off >= 1; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off));
    const float scale = block_scale(amax);
    uint8_t *qo = q + t * H + b * block;
    for (int64_t i = lane; i < block; i += kWave)
        qo[i] = static_cast<uint8_t>(e4m3_code(load_x(row + i) / scale));
    if (lane == 0)
        scales[t * nb + b] = scale;
}

// ---------------------------------------------------------------- fused dispatch
// Zero-fills padding rows (gather-map entries outside [0, src_rows), but not MOE_ROW_UNUSED):
// their codes and their scales.
__device__ __forceinline__ void fp8_zero_rows(int64_t src_rows, int64_t H, int64_t nb, const int32_t *__restrict__ src_row,
                                              int64_t N, int64_t first, uint8_t *__restrict__ dst,
                                              float *__restrict__ dst_scales)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i = first + lane;
    bool zero = false;
    if (src_row && lane < kFp8ZeroRows && i < N) {
        const int32_t s = src_row[i];
        zero = (s < 0 || s >= src_rows) && s != MOE_ROW_UNUSED;
    }
    uint64_t m = __ballot(zero);
    const __attribute__((ext_vector_type(2))) unsigned int z = {0u, 0u};
    while (m) {
        const int j = __builtin_ctzll(m);
        m &= m - 1;
        const __amdgpu_buffer_rsrc_t d = make_rsrc(dst + (first + j) * H, static_cast<uint32_t>(H));
        for (int64_t v = lane; v * 8 < H; v += kWave)  // H is a multiple of 8: the stores tile the row
            __builtin_amdgcn_raw_buffer_store_b64(z, d, static_cast<int>(v * 8), 0, kPolicyStreamStore);
        for (int64_t b = lane; b < nb; b += kWave)
            dst_scales[(first + j) * nb + b] = 0.0f;
    }
}

template <typename X>
__global__ __launch_bounds__(kFp8Threads) void permute_scatter_fp8_kernel(
    const X *__restrict__ src, int64_t src_rows, int64_t H, int block, const int32_t *__restrict__ dst_of, int J,
    const int32_t *__restrict__ src_row, int64_t N, uint8_t *__restrict__ dst, float *__restrict__ dst_scales,
    int64_t zero_waves, bool zero_first)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t spr = (H + kFp8Slice - 1) / kFp8Slice;  // slices (wavefronts) per source row
    const int64_t nb = H / block;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kFp8Waves +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int64_t copy_waves = src_rows * spr;
    if (zero_first ? gw < zero_waves : gw >= copy_waves) {
        fp8_zero_rows(src_rows, H, nb, src_row, N, (zero_first ? gw : gw - copy_waves) * kFp8ZeroRows, dst, dst_scales);
        return;
    }
    const int64_t cw = zero_first ? gw - zero_waves : gw;
    const int64_t t = cw / spr;
    if (t >= src_rows)  // the grid's last workgroup may hold waves past the last row
        return;
    const int64_t e0 = (cw - t * spr) * kFp8Slice + 16 * lane;  // this lane's 16 elements: two halves
    const bool have0 = e0 < H, have1 = e0 + 8 < H;  // H is a multiple of 8
    // the first 64 entries of dst_of that name a destination (a token has fewer than 64 in
    // practice; later chunks are walked below)
    int j0 = 0;
    int32_t my = -1;
    uint64_t m = 0;
    for (; j0 < J; j0 += kWave) {
        my = j0 + lane < J ? dst_of[t * J + j0 + lane] : -1;
        m = __ballot(my >= 0 && my < N);
        if (m)
            break;
    }
    if (m == 0)
        return;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = 0.0f;
    {
        float h0[8], h1[8];
        if (have0)
            load8x(src + t * H + e0, h0);
        if (have1)
            load8x(src + t * H + e0 + 8, h1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = have0 ? h0[i] : 0.0f;
            v[8 + i] = have1 ? h1[i] : 0.0f;
        }
    }
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a0 = fmaxf(a0, fabsf(v[i]));
        a1 = fmaxf(a1, fabsf(v[8 + i]));
    }
    if (block > 8) {  // one block spans both halves and block/16 consecutive lanes
        a0 = fmaxf(a0, a1);
        for (int off = 1; off < block / 16; off <<= 1)
            a0 = fmaxf(a0, __shfl_xor(a0, off));
        a1 = a0;
    }
    const float s0 = block_scale(a0), s1 = block_scale(a1);
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        c[h] = e4m3_pack4(v[4 * h] / s0, v[4 * h + 1] / s0, v[4 * h + 2] / s0, v[4 * h + 3] / s0);
        c[2 + h] = e4m3_pack4(v[8 + 4 * h] / s1, v[8 + 4 * h + 1] / s1, v[8 + 4 * h + 2] / s1, v[8 + 4 * h + 3] / s1);
    }
    // scales: with block 8 each half is a block; otherwise the block's first lane writes it
    const bool first_lane = block == 8 || (lane % (block / 16)) == 0;
    const int64_t b0 = e0 / block;
    const bool whole16 = H % 16 == 0;
    for (;;) {
        if (m == 0) {  // next chunk of 64 entries
            j0 += kWave;
            if (j0 >= J)
                break;
            my = j0 + lane < J ? dst_of[t * J + j0 + lane] : -1;
            m = __ballot(my >= 0 && my < N);
            continue;
        }
        const int j = __builtin_ctzll(m);
        m &= m - 1;
        const int64_t d = __builtin_amdgcn_readlane(my, j);
        const __amdgpu_buffer_rsrc_t q = make_rsrc(dst + d * H, static_cast<uint32_t>(H));
        if (whole16) {
            if (have0)
                st16_buf<kPolicyStreamStore>(q, static_cast<uint32_t>(e0), u32x4{c[0], c[1], c[2], c[3]});
        } else {
            const __attribute__((ext_vector_type(2))) unsigned int lo = {c[0], c[1]}, hi = {c[2], c[3]};
            if (have0)
                __builtin_amdgcn_raw_buffer_store_b64(lo, q, static_cast<int>(e0), 0, kPolicyStreamStore);
            if (have1)
                __builtin_amdgcn_raw_buffer_store_b64(hi, q, static_cast<int>(e0 + 8), 0, kPolicyStreamStore);
        }
        if (have0 && first_lane) {
            dst_scales[d * nb + b0] = s0;
            if (block == 8 && have1)
                dst_scales[d * nb + b0 + 1] = s1;
        }
    }
}

bool pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

}  // namespace
}  // namespace moe

extern "C" moe_status moe_quantize_fp8(const void *x, moe_dtype x_dt, int64_t T, int64_t H, int32_t block,
                                       uint8_t *q, float *scales, hipStream_t stream)
{
    using namespace moe;
    if (x_dt == MOE_FP8_E4M3)
        return MOE_ERR_UNSUPPORTED;
    if (T < 0 || H < 1 || block < 1 || H % block != 0 || (x_dt != MOE_F32 && x_dt != MOE_BF16))
        return MOE_ERR_INVALID;
    if (T == 0)
        return MOE_OK;
    if (!x || !q || !scales)
        return MOE_ERR_INVALID;
    const int64_t blocks = ceil_div(T * (H / block), kFp8Waves);
    if (blocks > 0x7fffffff || H > 0x7fffffffLL / 4)
        return MOE_ERR_UNSUPPORTED;
    if (x_dt == MOE_BF16)
        hipLaunchKernelGGL(quantize_fp8_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(kFp8Threads), 0,
                           stream, static_cast<const uint16_t *>(x), T, H, static_cast<int64_t>(block), q, scales);
    else
        hipLaunchKernelGGL(quantize_fp8_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(kFp8Threads), 0,
                           stream, static_cast<const float *>(x), T, H, static_cast<int64_t>(block), q, scales);
    return launch_status();
}

extern "C" moe_status moe_permute_scatter_fp8(const void *src, moe_dtype src_dt, int64_t src_rows, int64_t H,
                                              int32_t block, const int32_t *dst_of, int32_t J, const int32_t *src_row,
                                              int64_t N, uint8_t *dst, float *dst_scales, hipStream_t stream)
{
    using namespace moe;
    if (src_dt == MOE_FP8_E4M3)
        return MOE_ERR_UNSUPPORTED;
    if (src_rows < 0 || H < 1 || N < 0 || J < 1 || block < 1 || H % block != 0 ||
        (src_dt != MOE_F32 && src_dt != MOE_BF16))
        return MOE_ERR_INVALID;
    if (J > MOE_MAX_EXPERTS || !pow2(block) || block < 8 || block > kFp8Slice)
        return MOE_ERR_UNSUPPORTED;
    if (N == 0 || (src_rows == 0 && !src_row))
        return MOE_OK;
    if (!dst || !dst_scales || (src_rows > 0 && (!src || !dst_of)))
        return MOE_ERR_INVALID;
    if (H * 4 > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    if (!aligned16(dst) || (src_rows > 0 && !aligned16(src)))
        return MOE_ERR_UNSUPPORTED;
    const bool zero_first = src_row && N > src_rows * J;  // padding rows are certain: zero them first
    const int64_t zwaves = src_row ? ceil_div(N, kFp8ZeroRows) : 0;
    const int64_t blocks = ceil_div(src_rows * ceil_div(H, kFp8Slice) + zwaves, kFp8Waves);
    if (blocks > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    if (src_dt == MOE_BF16)
        hipLaunchKernelGGL(permute_scatter_fp8_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(kFp8Threads),
                           0, stream, static_cast<const uint16_t *>(src), src_rows, H, static_cast<int>(block), dst_of,
                           J, src_row, N, dst, dst_scales, zwaves, zero_first);
    else
        hipLaunchKernelGGL(permute_scatter_fp8_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(kFp8Threads), 0,
                           stream, static_cast<const float *>(src), src_rows, H, static_cast<int>(block), dst_of, J,
                           src_row, N, dst, dst_scales, zwaves, zero_first);
    return launch_status();
}
