// Unpermute + weighted top-k merge, and the per-group local pre-combine.
//
// [Combine] §1 ("03 · Combine 与 forward / backward 对称性"): out[t] = sum over the token's top-k
// experts of probs[t,e] * expert_e(x[t]). [Scratch] §13/§16 ("从零理解 MoE 算子"): unpermute is
// the inverse of the permute and output[token] = sum_k weight[token,k] * expert_output[token,k].
// [CANN] §1(2): the outputs of a token's experts on one rank are merged before leaving it.
//
// gfx950 design: a deterministic gather instead of an atomic scatter_add. One workgroup owns
// one token: it compacts the token's valid (row, weight) pairs into LDS in slot order, then
// every thread owns 8 consecutive hidden elements at a time, issues the 16-byte loads of all
// the token's rows before the fused multiply-adds (which run in slot order, float32, from +0),
// and writes 8 outputs with one 16-byte (bf16) or two (float32) stores. Each y row is read once
// and each out row written once, both with nontemporal hints (streamed data: no reuse to keep
// in L2 / MALL, which measurably raises the read rate on MI355X).
#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxCombineK = 1024;
constexpr int kMaxThreads = 1024;  // largest workgroup block_threads() picks
constexpr int kBatch = 8;  // rows whose loads are issued together

// ---------------------------------------------------------------- 8-element vector access
template <typename Y>
struct Vec8Load;

template <>
struct Vec8Load<uint16_t> {  // bf16: one 16-byte load
    __device__ static void load(const uint16_t *p, float (&v)[8])
    {
        const u32x4 q = ld16_stream(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
        v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
        v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
};

template <>
struct Vec8Load<float> {  // float32: two 16-byte loads
    __device__ static void load(const float *p, float (&v)[8])
    {
        const u32x4 a = ld16_stream(p), b = ld16_stream(p + 4);
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    }
};

__device__ __forceinline__ void store8(uint16_t *p, const float (&a)[8])
{
    st16_stream(p, u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
                         pack_bf16x2(a[6], a[7])});
}

__device__ __forceinline__ void store8(float *p, const float (&a)[8])
{
    st16_stream(p, u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]), __float_as_uint(a[3])});
    st16_stream(p + 4, u32x4{__float_as_uint(a[4]), __float_as_uint(a[5]), __float_as_uint(a[6]), __float_as_uint(a[7])});
}

__device__ __forceinline__ float load1(const uint16_t *p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ void store1(uint16_t *p, float a) { *p = static_cast<uint16_t>(f32_to_bf16_bits(a)); }
__device__ __forceinline__ void store1(float *p, float a) { *p = a; }

// acc = fma(w, y[rows[j]], acc) for j = 0..n-1 in order, 8 elements at column c8*8.
template <typename Y, bool VEC>
__device__ __forceinline__ void accumulate(const Y *__restrict__ y, int64_t H, const int32_t *rows,
                                           const float *ws, int n, int64_t col, float (&acc)[8])
{
    for (int j0 = 0; j0 < n; j0 += kBatch) {
        float v[kBatch][8];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (j0 + u < n) {
                const Y *p = y + static_cast<int64_t>(rows[j0 + u]) * H + col;
                if constexpr (VEC) {
                    Vec8Load<Y>::load(p, v[u]);
                } else {
                    v[u][0] = load1(p);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (j0 + u < n) {
                const float w = ws[j0 + u];
#pragma unroll
                for (int q = 0; q < (VEC ? 8 : 1); ++q)
                    acc[q] = __builtin_fmaf(w, v[u][q], acc[q]);
            }
        }
    }
}

// Compacts the valid entries of rows_in[0..K) (in order) into LDS; returns their number.
// Runs on wave 0; the caller synchronises.
__device__ int compact_rows(const int32_t *rows_in, const float *w_in, int K, int64_t y_rows,
                            int32_t *rows, float *ws, int *n_out)
{
    const int lane = threadIdx.x;
    int n = 0;
    for (int k0 = 0; k0 < K; k0 += kWave) {
        const int k = k0 + lane;
        const int32_t r = k < K ? rows_in[k] : -1;
        const bool ok = r >= 0 && r < y_rows;
        const uint64_t m = __ballot(ok);
        if (ok) {
            const int pos = n + __popcll(m & lanemask_lt());
            rows[pos] = r;
            ws[pos] = w_in ? w_in[k] : 1.0f;
        }
        n += __popcll(m);
    }
    if (lane == 0)
        *n_out = n;
    return n;
}

template <typename Y, typename O, bool VEC>
__global__ __launch_bounds__(kMaxThreads) void combine_kernel(const Y *__restrict__ y, int64_t y_rows, int64_t H,
                                                      const int32_t *__restrict__ row_of,
                                                      const float *__restrict__ w, int K,
                                                      O *__restrict__ out)
{
    __shared__ int32_t rows[kMaxCombineK];
    __shared__ float ws[kMaxCombineK];
    __shared__ int n_sh;
    const int64_t t = blockIdx.x;
    if (threadIdx.x < kWave)
        compact_rows(row_of + t * K, w ? w + t * K : nullptr, K, y_rows, rows, ws, &n_sh);
    __syncthreads();
    const int n = n_sh;
    constexpr int kE = VEC ? 8 : 1;
    const int64_t nchunk = H / kE;
    O *o = out + t * H;
    for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        accumulate<Y, VEC>(y, H, rows, ws, n, c * kE, acc);
        if constexpr (VEC)
            store8(o + c * kE, acc);
        else
            store1(o + c, acc[0]);
    }
}

// ---------------------------------------------------------------- group pre-combine
template <typename Y, bool VEC>
__global__ __launch_bounds__(kMaxThreads) void precombine_kernel(const Y *__restrict__ y, int64_t y_rows, int64_t H,
                                                         const int32_t *__restrict__ row_of,
                                                         const float *__restrict__ w,
                                                         const int32_t *__restrict__ topk_idx, int K,
                                                         int E, int gs, int G,
                                                         const int32_t *__restrict__ slot_of,
                                                         int64_t slots_cap, float *__restrict__ partials)
{
    __shared__ int32_t grp[MOE_MAX_TOPK];   // group of slot k, -1 if it adds nothing
    __shared__ int32_t rows[MOE_MAX_TOPK];
    __shared__ float ws[MOE_MAX_TOPK];
    __shared__ int32_t item_g[MOE_MAX_EXPERTS];  // present (group, slot) pairs of this token
    __shared__ int32_t item_s[MOE_MAX_EXPERTS];
    __shared__ int n_items_sh;
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid < K) {
        const int e = topk_idx[t * K + tid];
        const int32_t r = row_of[t * K + tid];
        const bool ok = e >= 0 && e < E && r >= 0 && r < y_rows;
        grp[tid] = ok ? e / gs : -1;
        rows[tid] = ok ? r : 0;
        ws[tid] = w ? w[t * K + tid] : 1.0f;
    }
    if (tid < kWave) {
        int n = 0;
        for (int g0 = 0; g0 < G; g0 += kWave) {
            const int g = g0 + tid;
            const int32_t s = g < G ? slot_of[t * G + g] : -1;
            const bool ok = s >= 0 && s < slots_cap;
            const uint64_t m = __ballot(ok);
            if (ok) {
                const int pos = n + __popcll(m & lanemask_lt());
                item_g[pos] = g;
                item_s[pos] = s;
            }
            n += __popcll(m);
        }
        if (tid == 0)
            n_items_sh = n;
    }
    __syncthreads();
    const int n_items = n_items_sh;
    constexpr int kE = VEC ? 8 : 1;
    const int64_t nchunk = H / kE;
    for (int it = 0; it < n_items; ++it) {
        const int g = item_g[it];
        float *o = partials + static_cast<int64_t>(item_s[it]) * H;
        for (int64_t c = tid; c < nchunk; c += blockDim.x) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < K; k0 += kBatch) {
                float v[kBatch][8];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    if (k0 + u < K && grp[k0 + u] == g) {
                        const Y *p = y + static_cast<int64_t>(rows[k0 + u]) * H + c * kE;
                        if constexpr (VEC)
                            Vec8Load<Y>::load(p, v[u]);
                        else
                            v[u][0] = load1(p);
                    }
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    if (k0 + u < K && grp[k0 + u] == g) {
#pragma unroll
                        for (int q = 0; q < kE; ++q)
                            acc[q] = __builtin_fmaf(ws[k0 + u], v[u][q], acc[q]);
                    }
                }
            }
            if constexpr (VEC)
                store8(o + c * kE, acc);
            else
                store1(o + c, acc[0]);
        }
    }
}

// Threads per token: about two 8-element chunks per thread, whole wavefronts, at most 1024
// (H = 7168 -> 448 threads, two chunks each).
int block_threads(int64_t nchunk)
{
    const int64_t half = (nchunk + 1) / 2;
    const int64_t waves = std::min<int64_t>(kMaxThreads / kWave, std::max<int64_t>(1, (half + kWave - 1) / kWave));
    return static_cast<int>(waves * kWave);
}

template <typename Y, typename O>
moe_status launch_combine(const void *y, int64_t y_rows, int64_t H, const int32_t *row_of, const float *w,
                          int64_t T, int K, void *out, hipStream_t stream)
{
    const bool vec = H % 8 == 0 && aligned16(out) && (y_rows == 0 || aligned16(y));
    const int64_t nchunk = vec ? H / 8 : H;
    const dim3 grid(static_cast<unsigned>(T)), block(block_threads(nchunk));
    if (vec)
        hipLaunchKernelGGL((combine_kernel<Y, O, true>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, K, static_cast<O *>(out));
    else
        hipLaunchKernelGGL((combine_kernel<Y, O, false>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, K, static_cast<O *>(out));
    return launch_status();
}

template <typename Y>
moe_status launch_precombine(const void *y, int64_t y_rows, int64_t H, const int32_t *row_of, const float *w,
                             const int32_t *topk_idx, int64_t T, int K, int E, int gs,
                             const int32_t *slot_of, int64_t slots_cap, float *partials, hipStream_t stream)
{
    const bool vec = H % 8 == 0 && aligned16(partials) && (y_rows == 0 || aligned16(y));
    const int64_t nchunk = vec ? H / 8 : H;
    const dim3 grid(static_cast<unsigned>(T)), block(block_threads(nchunk));
    const int G = E / gs;
    if (vec)
        hipLaunchKernelGGL((precombine_kernel<Y, true>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, topk_idx, K, E, gs, G, slot_of, slots_cap, partials);
    else
        hipLaunchKernelGGL((precombine_kernel<Y, false>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, topk_idx, K, E, gs, G, slot_of, slots_cap, partials);
    return launch_status();
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_unpermute_combine(const void *y, moe_dtype y_dt, int64_t y_rows, int64_t H,
                                            const int32_t *row_of, const float *w, int64_t T, int32_t K,
                                            void *out, moe_dtype out_dt, hipStream_t stream)
{
    using namespace moe;
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || (y_dt != MOE_F32 && y_dt != MOE_BF16) ||
        (out_dt != MOE_F32 && out_dt != MOE_BF16))
        return MOE_ERR_INVALID;
    if (K > kMaxCombineK)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!row_of || !out || (y_rows > 0 && !y))
        return MOE_ERR_INVALID;
    if (T > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    if (y_dt == MOE_BF16)
        return out_dt == MOE_BF16 ? launch_combine<uint16_t, uint16_t>(y, y_rows, H, row_of, w, T, K, out, stream)
                                  : launch_combine<uint16_t, float>(y, y_rows, H, row_of, w, T, K, out, stream);
    return out_dt == MOE_BF16 ? launch_combine<float, uint16_t>(y, y_rows, H, row_of, w, T, K, out, stream)
                              : launch_combine<float, float>(y, y_rows, H, row_of, w, T, K, out, stream);
}

extern "C" moe_status moe_group_precombine(const void *y, moe_dtype y_dt, int64_t y_rows, int64_t H,
                                           const int32_t *row_of, const float *w, const int32_t *topk_idx,
                                           int64_t T, int32_t K, int32_t E, int32_t group_size,
                                           const int32_t *slot_of, int64_t slots_cap, float *partials,
                                           hipStream_t stream)
{
    using namespace moe;
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || E < 1 || group_size < 1 || E % group_size != 0 ||
        slots_cap < 0 || (y_dt != MOE_F32 && y_dt != MOE_BF16))
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!row_of || !topk_idx || !slot_of || (slots_cap > 0 && !partials) || (y_rows > 0 && !y))
        return MOE_ERR_INVALID;
    if (T > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    if (y_dt == MOE_BF16)
        return launch_precombine<uint16_t>(y, y_rows, H, row_of, w, topk_idx, T, K, E, group_size, slot_of,
                                           slots_cap, partials, stream);
    return launch_precombine<float>(y, y_rows, H, row_of, w, topk_idx, T, K, E, group_size, slot_of, slots_cap,
                                    partials, stream);
}
