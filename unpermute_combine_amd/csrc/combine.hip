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
// and each out row written once, both with streaming cache policies (no reuse to keep in L2 /
// MALL, which measurably raises the read rate on MI355X); y rows are read through buffer
// resources, which give the sc0|nt policy and a hardware bounds check.
//
// Rows with 4-byte elements (float32 inputs or outputs: the pre-combine's partials, the group
// final sum) use a split lane layout instead: per 512-element unit of a row, lane j of a
// wavefront owns elements 4j..4j+3 and 256+4j..256+4j+3, so every load or store instruction of
// the wavefront covers one contiguous span (1 KiB of float32, 512 B of bf16). With 8 consecutive
// elements per lane a 32-byte float32 chunk takes two 16-byte instructions that each touch only
// half of every 128-byte line; on MI355X that ran the pre-combine ~12% and the final sum ~15%
// slower.
#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxCombineK = 1024;
constexpr int kMaxThreads = 1024;  // largest workgroup block_threads() picks
constexpr int kBatch = 8;     // rows whose loads are issued together
constexpr int kFewTerms = 4;  // tokens with at most this many terms take the two-chunk path

// ---------------------------------------------------------------- 8-element vector access
// Raw 16-byte vector of one 8-element bf16 chunk (rows with 4-byte elements take the split layout).
template <typename Y>
struct Chunk;

template <>
struct Chunk<uint16_t> {
    static constexpr int kVecs = 1;
    __device__ static void widen(const u32x4 (&q)[1], float (&v)[8])
    {
        v[0] = bf16_lo(q[0].x); v[1] = bf16_hi(q[0].x);
        v[2] = bf16_lo(q[0].y); v[3] = bf16_hi(q[0].y);
        v[4] = bf16_lo(q[0].z); v[5] = bf16_hi(q[0].z);
        v[6] = bf16_lo(q[0].w); v[7] = bf16_hi(q[0].w);
    }
};

// Loads chunk `col8` (8 elements) of row `row` of y; a negative row gives zeros without a
// memory access (a zero-size buffer resource).
template <typename Y>
__device__ __forceinline__ void load_chunk(const Y *__restrict__ y, int64_t H, int32_t row, int64_t col8,
                                           u32x4 (&q)[Chunk<Y>::kVecs])
{
    const uint32_t row_bytes = static_cast<uint32_t>(H * sizeof(Y));
    const __amdgpu_buffer_rsrc_t r = make_rsrc(y + static_cast<int64_t>(row < 0 ? 0 : row) * H, row < 0 ? 0u : row_bytes);
    const uint32_t off = static_cast<uint32_t>(col8 * 8 * sizeof(Y));
#pragma unroll
    for (int i = 0; i < Chunk<Y>::kVecs; ++i)
        q[i] = ld16_buf<kPolicyStreamLoad>(r, off + 16 * i);
}

__device__ __forceinline__ void store8(uint16_t *p, const float (&a)[8])
{
    st16_stream(p, u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
                         pack_bf16x2(a[6], a[7])});
}

__device__ __forceinline__ float load1(const uint16_t *p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ void store1(uint16_t *p, float a) { *p = static_cast<uint16_t>(f32_to_bf16_bits(a)); }
__device__ __forceinline__ void store1(float *p, float a) { *p = a; }

// One batch of up to kBatch terms, acc = fma(w[u], y[row[u]], acc) in order u = 0, 1, ...; a
// negative row is an absent term: it loads nothing (zero-size resource) and its FMA result is
// discarded, so no branch splits the batch and all its loads are in flight before the first FMA.
template <typename Y>
__device__ __forceinline__ void fma_batch(const Y *__restrict__ y, int64_t H, const int32_t (&row)[kBatch],
                                          const float (&w)[kBatch], int64_t col8, float (&acc)[8])
{
    u32x4 q[kBatch][Chunk<Y>::kVecs];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
        load_chunk<Y>(y, H, row[u], col8, q[u]);
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const bool live = row[u] >= 0;
        float v[8];
        Chunk<Y>::widen(q[u], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r = __builtin_fmaf(w[u], v[e], acc[e]);
            acc[e] = live ? r : acc[e];
        }
    }
}

// Two chunks (c, c2) of the same (at most N) terms with all their loads in flight before the
// first FMA; row1 marks the terms of chunk c2 (negative: nothing to load).
template <typename Y, int N>
__device__ __forceinline__ void fma_two(const Y *__restrict__ y, int64_t H, const int32_t (&row)[kBatch],
                                        const int32_t (&row1)[kBatch], const float (&w)[kBatch], int64_t c,
                                        int64_t c2, float (&acc)[8], float (&acc2)[8])
{
    static_assert(N <= kBatch, "at most one batch of terms");
    u32x4 q[N][Chunk<Y>::kVecs];
    u32x4 q2[N][Chunk<Y>::kVecs];
#pragma unroll
    for (int u = 0; u < N; ++u) {
        load_chunk<Y>(y, H, row[u], c, q[u]);
        load_chunk<Y>(y, H, row1[u], c2, q2[u]);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const bool live = row[u] >= 0;
        float v[8], v2[8];
        Chunk<Y>::widen(q[u], v);
        Chunk<Y>::widen(q2[u], v2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r = __builtin_fmaf(w[u], v[e], acc[e]);
            acc[e] = live ? r : acc[e];
            const float r2 = __builtin_fmaf(w[u], v2[e], acc2[e]);
            acc2[e] = live ? r2 : acc2[e];
        }
    }
}

// Terms j0 .. j0+kBatch-1 of the compacted list (LDS) into registers; uniform across the block.
__device__ __forceinline__ void batch_terms(const int32_t *rows, const float *ws, int n, int j0,
                                            int32_t (&row)[kBatch], float (&w)[kBatch])
{
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const bool live = j0 + u < n;
        row[u] = live ? __builtin_amdgcn_readfirstlane(rows[j0 + u]) : -1;
        w[u] = live ? ws[j0 + u] : 0.0f;
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
        const float wk = (k < K && w_in) ? w_in[k] : 1.0f;  // loaded beside r, not after it
        const bool ok = r >= 0 && r < y_rows;
        const uint64_t m = __ballot(ok);
        if (ok) {
            const int pos = n + __popcll(m & lanemask_lt());
            rows[pos] = r;
            ws[pos] = wk;
        }
        n += __popcll(m);
    }
    if (lane == 0)
        *n_out = n;
    return n;
}

// ---------------------------------------------------------------- split layout (4-byte rows)
constexpr int kUnit = 512;  // elements per wavefront and unit: two halves of 64 lanes x 4

// Four consecutive elements as loaded: 8 bytes of bf16 or 16 bytes of float32.
template <typename Y>
struct Part;

template <>
struct Part<uint16_t> {
    uint32_t a, b;
    __device__ static Part load(__amdgpu_buffer_rsrc_t r, int64_t e)
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(e * 2), 0, kPolicyStreamLoad);
        return Part{static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1])};
    }
    __device__ void widen(float *v) const
    {
        v[0] = bf16_lo(a); v[1] = bf16_hi(a); v[2] = bf16_lo(b); v[3] = bf16_hi(b);
    }
};

template <>
struct Part<float> {
    u32x4 q;
    __device__ static Part load(__amdgpu_buffer_rsrc_t r, int64_t e)
    {
        return Part{ld16_buf<kPolicyStreamLoad>(r, static_cast<uint32_t>(e * 4))};
    }
    __device__ void widen(float *v) const
    {
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    }
};

// Both parts (elements e0.. and e0+256..) of a row; a negative row loads nothing (zero-size
// resource) and reads as zeros; elements past H read as zeros (the resource's bound).
template <typename Y>
__device__ __forceinline__ void load_parts(const Y *__restrict__ y, int64_t H, int32_t row, int64_t e0, Part<Y> (&q)[2])
{
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(y + static_cast<int64_t>(row < 0 ? 0 : row) * H, row < 0 ? 0u : static_cast<uint32_t>(H * sizeof(Y)));
    q[0] = Part<Y>::load(r, e0);
    q[1] = Part<Y>::load(r, e0 + kUnit / 2);
}

// acc = fma(w[u], value, acc) over the batch in order u = 0, 1, ... for the terms selected by
// `take[u]` (all loads issued first, absent terms discarded by a select, as in fma_batch).
template <typename Y>
__device__ __forceinline__ void fma_parts(const Part<Y> (&q)[kBatch][2], const float (&w)[kBatch],
                                          const bool (&take)[kBatch], float (&acc)[8])
{
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        float v[8];
        q[u][0].widen(v);
        q[u][1].widen(v + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r = __builtin_fmaf(w[u], v[e], acc[e]);
            acc[e] = take[u] ? r : acc[e];
        }
    }
}

template <typename Y>
__device__ __forceinline__ void fma_batch_split(const Y *__restrict__ y, int64_t H, const int32_t (&row)[kBatch],
                                                const float (&w)[kBatch], int64_t e0, float (&acc)[8])
{
    Part<Y> q[kBatch][2];
    bool take[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        load_parts<Y>(y, H, row[u], e0, q[u]);
        take[u] = row[u] >= 0;
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
    fma_parts<Y>(q, w, take, acc);
}

// Stores the 8 results of one lane at elements e0.. and e0+256.. of row `o` (stores past the
// resource's size, i.e. past H, are dropped by the hardware), with cache policy POL.
template <int POL = kPolicyNontemporal>
__device__ __forceinline__ void store_parts(__amdgpu_buffer_rsrc_t o, int64_t e0, const float (&a)[8], uint16_t *)
{
    __attribute__((ext_vector_type(2))) unsigned int lo = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    __attribute__((ext_vector_type(2))) unsigned int hi = {pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])};
    __builtin_amdgcn_raw_buffer_store_b64(lo, o, static_cast<int>(e0 * 2), 0, POL);
    __builtin_amdgcn_raw_buffer_store_b64(hi, o, static_cast<int>((e0 + kUnit / 2) * 2), 0, POL);
}

template <int POL = kPolicyNontemporal>
__device__ __forceinline__ void store_parts(__amdgpu_buffer_rsrc_t o, int64_t e0, const float (&a)[8], float *)
{
    st16_buf<POL>(o, static_cast<uint32_t>(e0 * 4),
                  u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]), __float_as_uint(a[3])});
    st16_buf<POL>(o, static_cast<uint32_t>((e0 + kUnit / 2) * 4),
                  u32x4{__float_as_uint(a[4]), __float_as_uint(a[5]), __float_as_uint(a[6]), __float_as_uint(a[7])});
}

template <typename Y, typename O>
constexpr bool kSplit = sizeof(Y) == 4 || sizeof(O) == 4;

// acc += the 8 bias values of a bf16 chunk (the combine's final bias, one float32 addition each)
__device__ __forceinline__ void add_bias8(const uint16_t *b, float (&acc)[8])
{
    const u32x4 q[1] = {ld16(b)};
    float v[8];
    Chunk<uint16_t>::widen(q, v);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = acc[e] + v[e];
}

template <typename Y, typename O, bool VEC>
__global__ __launch_bounds__(kMaxThreads) void combine_kernel(const Y *__restrict__ y, int64_t y_rows, int64_t H,
                                                      const int32_t *__restrict__ row_of,
                                                      const float *__restrict__ w, int K,
                                                      O *__restrict__ out, const O *__restrict__ bias)
{
    __shared__ int32_t rows[kMaxCombineK];
    __shared__ float ws[kMaxCombineK];
    __shared__ int n_sh;
    const int64_t t = blockIdx.x;
    if (threadIdx.x < kWave)
        compact_rows(row_of + t * K, w ? w + t * K : nullptr, K, y_rows, rows, ws, &n_sh);
    __syncthreads();
    const int n = n_sh;
    O *o = out + t * H;
    if constexpr (VEC && kSplit<Y, O>) {
        const int lane = threadIdx.x & (kWave - 1);
        const int nwaves = blockDim.x / kWave;
        const int64_t units = ceil_div(H, kUnit);
        const __amdgpu_buffer_rsrc_t orr = make_rsrc(o, static_cast<uint32_t>(H * sizeof(O)));
        for (int64_t un = threadIdx.x / kWave; un < units; un += nwaves) {
            const int64_t e0 = un * kUnit + 4 * lane;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int j0 = 0; j0 < n; j0 += kBatch) {
                int32_t row[kBatch];
                float w[kBatch];
                batch_terms(rows, ws, n, j0, row, w);
                fma_batch_split<Y>(y, H, row, w, e0, acc);
            }
            if (bias) {
                Part<O> b[2];
                load_parts<O>(bias + t * H, H, 0, e0, b);
                float v[8];
                b[0].widen(v);
                b[1].widen(v + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[e] = acc[e] + v[e];
            }
            store_parts(orr, e0, acc, o);
        }
    } else if constexpr (VEC) {
        int32_t row0[kBatch];  // the first batch of terms stays in registers for every chunk
        float w0[kBatch];
        batch_terms(rows, ws, n, 0, row0, w0);
        const int64_t nchunk = H / 8;
        if (n > kFewTerms) {
            // many terms: one chunk per thread, the token's rows read whole and at once
            for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
                float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                fma_batch<Y>(y, H, row0, w0, c, acc);
                for (int j0 = kBatch; j0 < n; j0 += kBatch) {
                    int32_t row[kBatch];
                    float w[kBatch];
                    batch_terms(rows, ws, n, j0, row, w);
                    fma_batch<Y>(y, H, row, w, c, acc);
                }
                if (bias)
                    add_bias8(bias + t * H + c * 8, acc);
                store8(o + c * 8, acc);
            }
        } else {
            // few terms (n <= kFewTerms): two chunks per thread, the loads of both in flight
            // together (with a workgroup of one thread per chunk, half the threads have nothing
            // to do)
            const int64_t half = (nchunk + 1) / 2;
            for (int64_t c = threadIdx.x; c < half; c += blockDim.x) {
                const int64_t c2 = c + half;
                float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                float acc2[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                int32_t row1[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    row1[u] = c2 < nchunk ? row0[u] : -1;
                fma_two<Y, kFewTerms>(y, H, row0, row1, w0, c, c2, acc, acc2);
                if (bias) {
                    add_bias8(bias + t * H + c * 8, acc);
                    if (c2 < nchunk)
                        add_bias8(bias + t * H + c2 * 8, acc2);
                }
                store8(o + c * 8, acc);
                if (c2 < nchunk)
                    store8(o + c2 * 8, acc2);
            }
        }
    } else {
        for (int64_t h = threadIdx.x; h < H; h += blockDim.x) {
            float acc = 0.0f;
            for (int j = 0; j < n; ++j)
                acc = __builtin_fmaf(ws[j], load1(y + static_cast<int64_t>(rows[j]) * H + h), acc);
            if (bias)
                acc = acc + load1(bias + t * H + h);
            store1(o + h, acc);
        }
    }
}

// ---------------------------------------------------------------- batched combine (bf16, 5..8 slots)
// The same per-token arithmetic as combine_kernel, but one workgroup combines kCombineBatch
// tokens: their valid slots are compacted together (one barrier), tokens are accumulated two at a
// time (the 16-byte loads of both tokens' rows in flight together), the bf16 results wait in LDS,
// and the workgroup writes its tokens' rows in one burst at the end. Reads and writes then reach
// HBM in longer runs: at T16384 H7168 K8 the combine took 352 us instead of 365 us (without its
// stores it reads in 287 us -- the interleaved writes are what costs). A workgroup has one thread
// per two chunks, each thread taking its two chunks one after the other: 345 us against 355 us
// with one thread per chunk and 432 us with one per four. It needs enough workgroups to fill the
// chip: with T8192 (drop-and-pad, H4096, ~2.8 terms per token) it was slower, 65 us against
// 55 us, so it is used from kBatchMinGroups workgroups (8 per CU) up.
constexpr int kCombineBatch = 8;
constexpr int64_t kStageBudget = 128 * 1024;  // LDS bytes of staged output rows per workgroup
constexpr int64_t kBatchMinGroups = 2048;

__global__ __launch_bounds__(kMaxThreads) void combine_batched_kernel(const uint16_t *__restrict__ y, int64_t y_rows,
                                                              int64_t H, const int32_t *__restrict__ row_of,
                                                              const float *__restrict__ w, int K, int64_t T,
                                                              uint16_t *__restrict__ out,
                                                              const uint16_t *__restrict__ bias)
{
    extern __shared__ u32x4 stage[];  // [kCombineBatch][H / 8]
    __shared__ int32_t rows[kCombineBatch][kBatch];
    __shared__ float ws[kCombineBatch][kBatch];
    __shared__ int n_sh[kCombineBatch];
    const int64_t nchunk = H / 8;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kCombineBatch;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    for (int tb = wave; tb < kCombineBatch; tb += nwaves) {  // token tb's valid slots, in slot order (K <= 8)
        const int64_t t = t0 + tb;
        const int32_t r = (t < T && lane < K) ? row_of[t * K + lane] : -1;
        const float wk = (t < T && lane < K && w) ? w[t * K + lane] : 1.0f;  // loaded beside r
        const bool ok = r >= 0 && r < y_rows;
        const uint64_t m = __ballot(ok);
        if (ok) {
            const int pos = __popcll(m & lanemask_lt());
            rows[tb][pos] = r;
            ws[tb][pos] = wk;
        }
        if (lane == 0)
            n_sh[tb] = __popcll(m);
    }
    __syncthreads();
    for (int tb = 0; tb < kCombineBatch; tb += 2) {
        int32_t ra[kBatch], rb[kBatch];
        float wa[kBatch], wb[kBatch];
        batch_terms(rows[tb], ws[tb], n_sh[tb], 0, ra, wa);
        batch_terms(rows[tb + 1], ws[tb + 1], n_sh[tb + 1], 0, rb, wb);
        for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
            u32x4 qa[kBatch][1], qb[kBatch][1];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                load_chunk<uint16_t>(y, H, ra[u], c, qa[u]);
                load_chunk<uint16_t>(y, H, rb[u], c, qb[u]);
            }
            // (the compiler waits for the first row's load before issuing the other 15; a
            // scheduling barrier that issues all 16 first measured slower: 352 against 345 us)
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float acc2[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                float v[8], v2[8];
                Chunk<uint16_t>::widen(qa[u], v);
                Chunk<uint16_t>::widen(qb[u], v2);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float r = __builtin_fmaf(wa[u], v[e], acc[e]);
                    acc[e] = ra[u] >= 0 ? r : acc[e];
                    const float r2 = __builtin_fmaf(wb[u], v2[e], acc2[e]);
                    acc2[e] = rb[u] >= 0 ? r2 : acc2[e];
                }
            }
            if (bias) {
                if (t0 + tb < T)
                    add_bias8(bias + (t0 + tb) * H + c * 8, acc);
                if (t0 + tb + 1 < T)
                    add_bias8(bias + (t0 + tb + 1) * H + c * 8, acc2);
            }
            stage[tb * nchunk + c] = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                           pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
            stage[(tb + 1) * nchunk + c] = u32x4{pack_bf16x2(acc2[0], acc2[1]), pack_bf16x2(acc2[2], acc2[3]),
                                                 pack_bf16x2(acc2[4], acc2[5]), pack_bf16x2(acc2[6], acc2[7])};
        }
    }
    __syncthreads();
    for (int tb = 0; tb < kCombineBatch; ++tb) {
        const int64_t t = t0 + tb;
        if (t >= T)
            break;
        // sc1|nt through a row resource: the combine's own time is unchanged against plain
        // nontemporal stores, the whole step 0.705 -> 0.703 ms (T16384 H7168 K8)
        const __amdgpu_buffer_rsrc_t orow = make_rsrc(out + t * H, static_cast<uint32_t>(H * 2));
        for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x)
            st16_buf<kPolicyStreamStore>(orow, static_cast<uint32_t>(c * 16), stage[tb * nchunk + c]);
    }
}

// ---------------------------------------------------------------- group pre-combine
// Store policy of the partials: device-scope stores that keep the normal (temporal) cache policy.
// Every store instruction covers whole lines (1 KiB of float32, 512 B of bf16), and measured with
// caches flushed at T8192 H7168 (32 groups of 8) the pre-combine took 255 us against 284 us with
// nontemporal or sc1|nt stores (264 us with plain or sc0 stores), the final sum that reads the
// partials 138 instead of 131 us: the step 0.746 -> 0.732 ms. With bf16 partials the pre-combine
// took 213 instead of 222 us and the final sum 70 instead of 73 us (step 0.627 -> 0.612 ms).
constexpr int kPartialsStore = kPolicyDeviceStore;

template <typename Y, typename P, bool VEC>
__global__ __launch_bounds__(kMaxThreads) void precombine_kernel(const Y *__restrict__ y, int64_t y_rows, int64_t H,
                                                         const int32_t *__restrict__ row_of,
                                                         const float *__restrict__ w,
                                                         const int32_t *__restrict__ topk_idx, int K,
                                                         int E, int gs, int G,
                                                         const int32_t *__restrict__ slot_of,
                                                         int64_t slots_cap, P *__restrict__ partials)
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
    if constexpr (VEC) {
        const int lane = tid & (kWave - 1);
        const int nwaves = blockDim.x / kWave;
        const int64_t units = ceil_div(H, kUnit);
        if (K <= kBatch) {
            // every slot of the token in one batch: its rows are loaded once per unit and each
            // (group, slot) partial is reduced from registers
            int32_t row[kBatch];
            float wv[kBatch];
            int32_t gk[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const bool live = u < K && grp[u] >= 0;
                row[u] = live ? __builtin_amdgcn_readfirstlane(rows[u]) : -1;
                wv[u] = live ? ws[u] : 0.0f;
                gk[u] = live ? grp[u] : -1;
            }
            for (int64_t un = tid / kWave; un < units; un += nwaves) {
                const int64_t e0 = un * kUnit + 4 * lane;
                Part<Y> q[kBatch][2];
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    load_parts<Y>(y, H, row[u], e0, q[u]);
                for (int it = 0; it < n_items; ++it) {
                    const int g = item_g[it];
                    bool take[kBatch];
#pragma unroll
                    for (int u = 0; u < kBatch; ++u)
                        take[u] = gk[u] == g;
                    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                    fma_parts<Y>(q, wv, take, acc);
                    const int32_t s = __builtin_amdgcn_readfirstlane(item_s[it]);
                    store_parts<kPartialsStore>(
                        make_rsrc(partials + static_cast<int64_t>(s) * H, static_cast<uint32_t>(H * sizeof(P))), e0, acc,
                        partials);
                }
            }
        } else {
            for (int64_t un = tid / kWave; un < units; un += nwaves) {
                const int64_t e0 = un * kUnit + 4 * lane;
                for (int it = 0; it < n_items; ++it) {
                    const int g = item_g[it];
                    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                    for (int k0 = 0; k0 < K; k0 += kBatch) {
                        int32_t row[kBatch];
                        float w[kBatch];
#pragma unroll
                        for (int u = 0; u < kBatch; ++u) {
                            const bool member = k0 + u < K && grp[k0 + u] == g;
                            row[u] = member ? __builtin_amdgcn_readfirstlane(rows[k0 + u]) : -1;
                            w[u] = member ? ws[k0 + u] : 0.0f;
                        }
                        fma_batch_split<Y>(y, H, row, w, e0, acc);
                    }
                    const int32_t s = __builtin_amdgcn_readfirstlane(item_s[it]);
                    store_parts<kPartialsStore>(
                        make_rsrc(partials + static_cast<int64_t>(s) * H, static_cast<uint32_t>(H * sizeof(P))), e0, acc,
                        partials);
                }
            }
        }
    } else {
        for (int it = 0; it < n_items; ++it) {
            const int g = item_g[it];
            P *o = partials + static_cast<int64_t>(item_s[it]) * H;
            for (int64_t h = tid; h < H; h += blockDim.x) {
                float acc = 0.0f;
                for (int k = 0; k < K; ++k) {
                    const bool member = grp[k] == g;
                    const float v = member ? load1(y + static_cast<int64_t>(rows[k]) * H + h) : 0.0f;
                    const float r = __builtin_fmaf(member ? ws[k] : 0.0f, v, acc);
                    acc = member ? r : acc;
                }
                store1(o + h, acc);
            }
        }
    }
}

// ---------------------------------------------------------------- combine backward
// [Combine] §4: the combine is linear in the expert outputs, so its backward is the transposed
// map -- a dispatch of the output gradient back to the expert rows, scaled by the weights -- and
// the weights' gradient is a row dot product:
//   dy[row_of[t,k]] = w[t,k] * dout[t]      (float32 product, stored as float32 or bf16)
//   dw[t,k]         = <dout[t], y[row_of[t,k]]>
// One workgroup per token. Each thread owns 8 elements at a time (chunk layout for bf16-only
// rows, split layout as soon as one side is float32): it loads its part of dout[t] once, and per
// batch of 8 slots issues the loads of the same part of their y rows, then stores w*dout to each
// dy row before it uses the y values -- the stores leave while the loads are in flight (issuing
// them after the dot products took 896 us instead of 732 us at T16384 H7168 K8 bf16) -- and
// accumulates one partial dot per slot. The partial dots are reduced in a fixed order: per lane
// over its chunks in order, each chunk's 8 products in order; then over the wavefront by a
// reduce-scatter butterfly (xor 32, 16 and 8 each hand half of the remaining slots to the
// partner, then xor 4, 2, 1 on the one slot left, so that lanes 8u..8u+7 hold slot u's sum: 10
// exchanges instead of 48); then the wavefronts in order. The result is deterministic. An absent
// slot (row outside [0, y_rows)) has a zero-size resource: its loads read 0 and its stores are
// dropped, and its dw is 0. Workgroups past the last token zero the rows of dy that the gather
// map src_row leaves without a source (padding rows).
//
// With bf16 dout, y and dy the call takes two passes instead: dy = w * dout is the source-major
// scatter of dout through row_of with a per-destination weight (the permute's kernel and launch
// shape; its padding waves zero the padding rows), then this kernel with its stores compiled out
// computes dw, reading dout and y only. A kernel that loads, stores and reduces at once mixes
// the HBM read and write streams within every wavefront; the two passes each keep one direction
// dominant. Measured with caches flushed: T16384 H7168 K8 743 -> 697 us, T8192 H7168 (32 groups
// of 8) 374 -> 356 us, T4096 H4096 K2 51.5 -> 47.5 us, drop-and-pad T8192 H4096 E128 195 -> 194 us;
// two workgroups per token (four slots each, dout read by both) lost instead (804 and 259 us).
// The dots pass runs first. It loads dout with the default policy and y with streaming loads, so
// most of dout is still in the 256 MB MALL when the scatter reads it again: the scatter, whose
// short waves wait on that read, then took 119 instead of 131 us at drop-and-pad T8192 H4096
// E128 and 321 instead of 351 us at T16384 H7168 K8, the dots 2 and 12 us more than when they
// came second (the call 174 -> 165 us and 644 -> 626 us; in group mode T8192 H7168 328 -> 319 us).
// Running the dots concurrently on a second stream lost (197 against 180 us by the events).
constexpr int kBwdZeroRowsPerWave = 16;

template <bool SPLIT>
__device__ __forceinline__ int64_t chunk_e0(int64_t c)
{
    return SPLIT ? (c / kWave) * kUnit + 4 * (c % kWave) : 8 * c;
}

template <typename X, bool SPLIT, int AUX = kPolicyStreamLoad>
__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, int64_t e0, float (&v)[8])
{
    if constexpr (SPLIT) {
        const Part<X> a = Part<X>::load(r, e0);
        const Part<X> b = Part<X>::load(r, e0 + kUnit / 2);
        a.widen(v);
        b.widen(v + 4);
    } else {
        const u32x4 q[1] = {ld16_buf<AUX>(r, static_cast<uint32_t>(e0 * 2))};
        Chunk<uint16_t>::widen(q, v);
    }
}

template <typename X, bool SPLIT>
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, int64_t e0, const float (&a)[8])
{
    if constexpr (SPLIT) {
        store_parts(r, e0, a, static_cast<X *>(nullptr));
    } else {
        st16_buf<kPolicyStreamStore>(r, static_cast<uint32_t>(e0 * 2),
                                     u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
                                           pack_bf16x2(a[6], a[7])});
    }
}

// Sums p[u] over the workgroup (fixed order, see above) and lets threads u < n write
// dw[u] (0 for an absent slot). Ends with a barrier, so `red` can be reused.
__device__ __forceinline__ void reduce_dots(float (&p)[kBatch], float (*red)[kBatch], int n, const int32_t *rows,
                                            int64_t y_rows, float *dw)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
    float a4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float send = b5 ? p[i] : p[4 + i];
        const float keep = b5 ? p[4 + i] : p[i];
        a4[i] = keep + __shfl_xor(send, 32);
    }
    float a2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = b4 ? a4[i] : a4[2 + i];
        const float keep = b4 ? a4[2 + i] : a4[i];
        a2[i] = keep + __shfl_xor(send, 16);
    }
    float a1 = (b3 ? a2[1] : a2[0]) + __shfl_xor(b3 ? a2[0] : a2[1], 8);
    a1 += __shfl_xor(a1, 4);
    a1 += __shfl_xor(a1, 2);
    a1 += __shfl_xor(a1, 1);
    if ((lane & 7) == 0)
        red[wave][lane >> 3] = a1;  // slot lane/8
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < n) {
        float s = 0.0f;
        for (int q = 0; q < static_cast<int>(blockDim.x / kWave); ++q)
            s += red[q][threadIdx.x];
        const int32_t r = rows[threadIdx.x];
        dw[threadIdx.x] = (r >= 0 && r < y_rows) ? s : 0.0f;
    }
    __syncthreads();
}

// reduce_dots for a compacted list of n slots: p[u] belongs to slot ks[u]; thread u < n writes
// dw[ks[u]] (the slots left out were written by the caller).
__device__ __forceinline__ void reduce_dots_compact(float (&p)[kBatch], float (*red)[kBatch], int n, const int *ks,
                                                    float *dw)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
    float a4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float send = b5 ? p[i] : p[4 + i];
        const float keep = b5 ? p[4 + i] : p[i];
        a4[i] = keep + __shfl_xor(send, 32);
    }
    float a2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = b4 ? a4[i] : a4[2 + i];
        const float keep = b4 ? a4[2 + i] : a4[i];
        a2[i] = keep + __shfl_xor(send, 16);
    }
    float a1 = (b3 ? a2[1] : a2[0]) + __shfl_xor(b3 ? a2[0] : a2[1], 8);
    a1 += __shfl_xor(a1, 4);
    a1 += __shfl_xor(a1, 2);
    a1 += __shfl_xor(a1, 1);
    if ((lane & 7) == 0)
        red[wave][lane >> 3] = a1;
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < n) {
        float sum = 0.0f;
        for (int q = 0; q < static_cast<int>(blockDim.x / kWave); ++q)
            sum += red[q][threadIdx.x];
        dw[ks[threadIdx.x]] = sum;
    }
}

template <typename D, typename Y, typename DY, bool SPLIT, bool DW, bool STORE = true>
__global__ __launch_bounds__(kMaxThreads) void combine_backward_kernel(
    const D *__restrict__ dout, const Y *__restrict__ y, int64_t y_rows, int64_t H, const int32_t *__restrict__ row_of,
    const float *__restrict__ w, int K, int64_t T, const int32_t *__restrict__ src_row, DY *__restrict__ dy,
    float *__restrict__ dw)
{
    __shared__ float red[kMaxThreads / kWave][kBatch];
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    const uint32_t dy_bytes = static_cast<uint32_t>(H * sizeof(DY));
    const int64_t t = blockIdx.x;
    if (t >= T) {
        const int64_t first = ((t - T) * nwaves + threadIdx.x / kWave) * kBwdZeroRowsPerWave;
        const int64_t i = first + lane;
        const bool zero = lane < kBwdZeroRowsPerWave && i < y_rows && (src_row[i] < 0 || src_row[i] >= T) && src_row[i] != MOE_ROW_UNUSED;
        uint64_t m = __ballot(zero);
        const u32x4 z{0u, 0u, 0u, 0u};
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            const __amdgpu_buffer_rsrc_t d = make_rsrc(dy + (first + j) * H, dy_bytes);
            for (uint32_t off = lane * 16u; off < dy_bytes; off += kWave * 16u)
                st16_buf<kPolicyStreamStore>(d, off, z);
        }
        return;
    }
    const int64_t nchunk = SPLIT ? ceil_div(H, kUnit) * kWave : H / 8;
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dout + t * H, static_cast<uint32_t>(H * sizeof(D)));
    const uint32_t y_bytes = static_cast<uint32_t>(H * sizeof(Y));
    if constexpr (DW && !STORE && !SPLIT) {
        // the dots pass of bf16 rows: a token's live slots compacted; with at most kFewTerms of
        // them (drop-and-pad keeps ~3 of 8) every thread takes two chunks with all their loads in
        // flight together, as the combine does for few terms
        __shared__ int32_t live_row[kBatch];
        __shared__ int live_k[kBatch];
        __shared__ int n_live_sh;
        if (K <= kBatch) {
            if (threadIdx.x < kWave) {
                const int k = threadIdx.x;
                const int32_t r = k < K ? row_of[t * K + k] : -1;
                const bool ok = r >= 0 && r < y_rows;
                const uint64_t m = __ballot(ok);
                if (ok) {
                    const int pos = __popcll(m & lanemask_lt());
                    live_row[pos] = r;
                    live_k[pos] = k;
                }
                if (k < K && !ok)
                    dw[t * K + k] = 0.0f;  // a slot that adds nothing
                if (k == 0)
                    n_live_sh = __popcll(m);
            }
            __syncthreads();
            const int n = n_live_sh;
            if (n <= kFewTerms) {
                int32_t rb[kFewTerms];
#pragma unroll
                for (int u = 0; u < kFewTerms; ++u)
                    rb[u] = u < n ? __builtin_amdgcn_readfirstlane(live_row[u]) : -1;
                float p[kBatch] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                const int64_t half = (nchunk + 1) / 2;
                for (int64_t c = threadIdx.x; c < half; c += blockDim.x) {
                    const int64_t c2 = c + half;
                    const bool has2 = c2 < nchunk;
                    float d[8], d2[8], yv[kFewTerms][8], y2[kFewTerms][8];
                    load8<D, false, 0>(dr, 8 * c, d);
                    load8<D, false, 0>(dr, 8 * c2, d2);  // past the row: reads zeros, unused
#pragma unroll
                    for (int u = 0; u < kFewTerms; ++u) {
                        const __amdgpu_buffer_rsrc_t yr =
                            make_rsrc(y + static_cast<int64_t>(rb[u] < 0 ? 0 : rb[u]) * H, rb[u] < 0 ? 0u : y_bytes);
                        load8<Y, false>(yr, 8 * c, yv[u]);
                        load8<Y, false>(yr, 8 * c2, y2[u]);
                    }
#pragma unroll
                    for (int u = 0; u < kFewTerms; ++u) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            p[u] = __builtin_fmaf(d[e], yv[u][e], p[u]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float r2 = __builtin_fmaf(d2[e], y2[u][e], p[u]);
                            p[u] = has2 ? r2 : p[u];
                        }
                    }
                }
                reduce_dots_compact(p, red, n, live_k, dw + t * K);
                return;
            }
        }
    }
    for (int k0 = 0; k0 < K; k0 += kBatch) {
        int32_t rb[kBatch];
        float wb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int k = k0 + u;
            const int32_t r = k < K ? row_of[t * K + k] : -1;
            rb[u] = (r >= 0 && r < y_rows) ? r : -1;
            wb[u] = (k < K && w) ? w[t * K + k] : 1.0f;
        }
        float p[kBatch] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
            const int64_t e0 = chunk_e0<SPLIT>(c);
            float d[8];
            load8<D, SPLIT, 0>(dr, e0, d);  // plain load: measured faster than streaming here
            float yv[kBatch][8];
            if constexpr (DW) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    load8<Y, SPLIT>(make_rsrc(y + static_cast<int64_t>(rb[u] < 0 ? 0 : rb[u]) * H, rb[u] < 0 ? 0u : y_bytes),
                                    e0, yv[u]);
            }
            if constexpr (STORE) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    float o[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        o[e] = wb[u] * d[e];
                    store8<DY, SPLIT>(make_rsrc(dy + static_cast<int64_t>(rb[u] < 0 ? 0 : rb[u]) * H, rb[u] < 0 ? 0u : dy_bytes),
                                      e0, o);
                }
            }
            if constexpr (DW) {
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        p[u] = __builtin_fmaf(d[e], yv[u][e], p[u]);
            }
        }
        if constexpr (DW)
            reduce_dots(p, red, K - k0 < kBatch ? K - k0 : kBatch, row_of + t * K + k0, y_rows, dw + t * K + k0);
    }
}

// Element-wise form (H not a multiple of 8, or unaligned rows): same arithmetic, one element
// per thread at a time, the dot reduced as above.
template <typename D, typename Y, typename DY>
__global__ __launch_bounds__(kMaxThreads) void combine_backward_scalar_kernel(
    const D *__restrict__ dout, const Y *__restrict__ y, int64_t y_rows, int64_t H, const int32_t *__restrict__ row_of,
    const float *__restrict__ w, int K, int64_t T, const int32_t *__restrict__ src_row, DY *__restrict__ dy,
    float *__restrict__ dw)
{
    __shared__ float red[kMaxThreads / kWave][kBatch];
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    const int64_t t = blockIdx.x;
    if (t >= T) {
        const int64_t first = ((t - T) * nwaves + threadIdx.x / kWave) * kBwdZeroRowsPerWave;
        const int64_t i = first + lane;
        const bool zero = lane < kBwdZeroRowsPerWave && i < y_rows && (src_row[i] < 0 || src_row[i] >= T) && src_row[i] != MOE_ROW_UNUSED;
        uint64_t m = __ballot(zero);
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            for (int64_t h = lane; h < H; h += kWave)
                store1(dy + (first + j) * H + h, 0.0f);
        }
        return;
    }
    for (int k0 = 0; k0 < K; k0 += kBatch) {
        float p[kBatch] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int k = k0 + u;
            const int32_t r = k < K ? row_of[t * K + k] : -1;
            if (r < 0 || r >= y_rows)
                continue;
            const float wk = w ? w[t * K + k] : 1.0f;
            for (int64_t h = threadIdx.x; h < H; h += blockDim.x) {
                const float d = load1(dout + t * H + h);
                store1(dy + static_cast<int64_t>(r) * H + h, wk * d);
                if (dw)
                    p[u] = __builtin_fmaf(d, load1(y + static_cast<int64_t>(r) * H + h), p[u]);
            }
        }
        if (dw)
            reduce_dots(p, red, K - k0 < kBatch ? K - k0 : kBatch, row_of + t * K + k0, y_rows, dw + t * K + k0);
    }
}

// Threads per workgroup: one per `cpt` 8-element chunks, whole wavefronts, at most 1024.
// Measured on MI355X (bf16 per-token combine): with at most 8 slots per token a workgroup of one
// thread per two chunks is faster for every mix of terms (for more slots, see launch_combine) -- T8192 H7168 with 8 terms 178 vs 185
// us, 6 terms (T4096) 70 vs 78 us, drop-and-pad T8192 H4096 E128 48 vs 56 us, K = 2 (T4096
// H4096) 24 vs 27 us; loading both chunks of a many-term token together instead of one after
// the other raised the registers to 112 (occupancy 4) and lost on the few-term tokens.
int block_threads(int64_t nchunk, int cpt)
{
    const int64_t per = (nchunk + cpt - 1) / cpt;
    const int64_t waves = std::min<int64_t>(kMaxThreads / kWave, std::max<int64_t>(1, (per + kWave - 1) / kWave));
    return static_cast<int>(waves * kWave);
}

// Threads per workgroup of the split layout: one wavefront per two 512-element units (taken one
// after the other), at most 1024. Measured at T8192 H7168 (32 groups of 8): pre-combine 288 us
// against 298 us with one wavefront per unit and 303 us with one per four.
int split_threads(int64_t H)
{
    return static_cast<int>(std::min<int64_t>(kMaxThreads / kWave, ceil_div(ceil_div(H, kUnit), 2)) * kWave);
}

template <typename Y, typename O>
moe_status launch_combine(const void *y, int64_t y_rows, int64_t H, const int32_t *row_of, const float *w,
                          const void *bias, int64_t T, int K, void *out, hipStream_t stream)
{
    const bool vec = H % 8 == 0 && aligned16(out) && (y_rows == 0 || aligned16(y)) && (!bias || aligned16(bias));
    const int64_t nchunk = vec ? H / 8 : H;
    // per-token kernel, bf16 rows: a workgroup of one thread per two chunks. For K > 8 this
    // favours sparse rows (the group final sum over bf16 partials, K = 32 with ~3 terms: 86 ->
    // 76 us) over dense ones (T4096 H4096 K = 32, every slot valid: 182 -> 191 us).
    const bool two = vec && !kSplit<Y, O>;
    const dim3 grid(static_cast<unsigned>(T)),
        block(vec && kSplit<Y, O> ? split_threads(H) : block_threads(nchunk, two ? 2 : 1));
    if constexpr (!kSplit<Y, O>) {
        const int64_t stage = static_cast<int64_t>(kCombineBatch) * H * 2;
        if (vec && K > kFewTerms && K <= kBatch && stage <= kStageBudget && ceil_div(T, kCombineBatch) >= kBatchMinGroups) {
            hipLaunchKernelGGL(combine_batched_kernel, dim3(static_cast<unsigned>(ceil_div(T, kCombineBatch))),
                               dim3(block_threads(nchunk, 2)),
                               static_cast<size_t>(stage), stream, static_cast<const uint16_t *>(y), y_rows, H, row_of,
                               w, K, T, static_cast<uint16_t *>(out), static_cast<const uint16_t *>(bias));
            return launch_status();
        }
    }
    if (vec)
        hipLaunchKernelGGL((combine_kernel<Y, O, true>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, K, static_cast<O *>(out), static_cast<const O *>(bias));
    else
        hipLaunchKernelGGL((combine_kernel<Y, O, false>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, K, static_cast<O *>(out), static_cast<const O *>(bias));
    return launch_status();
}

template <typename Y, typename P>
moe_status launch_precombine(const void *y, int64_t y_rows, int64_t H, const int32_t *row_of, const float *w,
                             const int32_t *topk_idx, int64_t T, int K, int E, int gs,
                             const int32_t *slot_of, int64_t slots_cap, void *partials, hipStream_t stream)
{
    const bool vec = H % 8 == 0 && (slots_cap == 0 || aligned16(partials)) && (y_rows == 0 || aligned16(y));
    const dim3 grid(static_cast<unsigned>(T)), block(vec ? split_threads(H) : block_threads(H, 2));
    const int G = E / gs;
    if (vec)
        hipLaunchKernelGGL((precombine_kernel<Y, P, true>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, topk_idx, K, E, gs, G, slot_of, slots_cap, static_cast<P *>(partials));
    else
        hipLaunchKernelGGL((precombine_kernel<Y, P, false>), grid, block, 0, stream, static_cast<const Y *>(y),
                           y_rows, H, row_of, w, topk_idx, K, E, gs, G, slot_of, slots_cap, static_cast<P *>(partials));
    return launch_status();
}

template <typename D, typename Y, typename DY>
moe_status launch_combine_backward(const void *dout, const void *y, int64_t y_rows, int64_t H, const int32_t *row_of,
                                   const float *w, int64_t T, int K, const int32_t *src_row, void *dy, float *dw,
                                   hipStream_t stream)
{
    constexpr bool split = sizeof(D) == 4 || sizeof(Y) == 4 || sizeof(DY) == 4;
    const bool vec = H % 8 == 0 && (T == 0 || aligned16(dout)) && (y_rows == 0 || aligned16(dy)) &&
                     (!dw || y_rows == 0 || aligned16(y));
    if constexpr (sizeof(D) == 2 && sizeof(Y) == 2 && sizeof(DY) == 2) {
        if (vec && K <= MOE_MAX_EXPERTS && H * 2 <= 0x7fffffffLL) {
            // bf16 rows: dy = w * dout is the weighted source-major scatter of dout through row_of
            // (which also zero-fills the padding rows named by src_row), and dw is a read-only pass
            // of dots launched before it; the two take their own best access patterns (see the
            // section comment) instead of one kernel that loads, stores and reduces together
            if (dw && T > 0) {  // the dots first: see the section comment
                const int threads = block_threads(H / 8, K <= kBatch ? 2 : 1);
                hipLaunchKernelGGL((combine_backward_kernel<D, Y, DY, false, true, false>), dim3(static_cast<unsigned>(T)),
                                   dim3(threads), 0, stream, static_cast<const D *>(dout), static_cast<const Y *>(y),
                                   y_rows, H, row_of, w, K, T, nullptr, static_cast<DY *>(dy), dw);
                const moe_status st = launch_status();
                if (st != MOE_OK)
                    return st;
            }
            return launch_scatter_vec16(static_cast<const char *>(dout), T, H * 2 / 16, row_of, K, src_row, y_rows,
                                        static_cast<char *>(dy), true, w, stream);
        }
    }
    // bf16 rows, at most kBatch slots: one thread per two chunks (taken one after the other);
    // measured 217 -> 190 us (drop-and-pad T8192 H4096 E128), 713 -> 700 us (T16384 H7168 K8)
    const int threads = vec ? (split ? split_threads(H) : block_threads(H / 8, K <= kBatch ? 2 : 1)) : block_threads(H, 1);
    const int64_t zero_blocks = src_row ? ceil_div(ceil_div(y_rows, kBwdZeroRowsPerWave), threads / kWave) : 0;
    const int64_t blocks = T + zero_blocks;
    if (blocks > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    if (blocks == 0)
        return MOE_OK;
    const dim3 grid(static_cast<unsigned>(blocks)), block(threads);
    if (vec && dw)
        hipLaunchKernelGGL((combine_backward_kernel<D, Y, DY, split, true>), grid, block, 0, stream,
                           static_cast<const D *>(dout), static_cast<const Y *>(y), y_rows, H, row_of, w, K, T, src_row,
                           static_cast<DY *>(dy), dw);
    else if (vec)
        hipLaunchKernelGGL((combine_backward_kernel<D, Y, DY, split, false>), grid, block, 0, stream,
                           static_cast<const D *>(dout), static_cast<const Y *>(y), y_rows, H, row_of, w, K, T, src_row,
                           static_cast<DY *>(dy), dw);
    else
        hipLaunchKernelGGL((combine_backward_scalar_kernel<D, Y, DY>), grid, block, 0, stream,
                           static_cast<const D *>(dout), static_cast<const Y *>(y), y_rows, H, row_of, w, K, T, src_row,
                           static_cast<DY *>(dy), dw);
    return launch_status();
}

template <typename D, typename Y>
moe_status launch_combine_backward_dy(moe_dtype dy_dt, const void *dout, const void *y, int64_t y_rows, int64_t H,
                                      const int32_t *row_of, const float *w, int64_t T, int K, const int32_t *src_row,
                                      void *dy, float *dw, hipStream_t stream)
{
    return dy_dt == MOE_BF16
               ? launch_combine_backward<D, Y, uint16_t>(dout, y, y_rows, H, row_of, w, T, K, src_row, dy, dw, stream)
               : launch_combine_backward<D, Y, float>(dout, y, y_rows, H, row_of, w, T, K, src_row, dy, dw, stream);
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_unpermute_combine(const void *y, moe_dtype y_dt, int64_t y_rows, int64_t H,
                                            const int32_t *row_of, const float *w, const void *bias, int64_t T,
                                            int32_t K, void *out, moe_dtype out_dt, hipStream_t stream)
{
    using namespace moe;
    if (y_dt == MOE_FP8_E4M3 || out_dt == MOE_FP8_E4M3)
        return MOE_ERR_UNSUPPORTED;  // the combine stays in bf16 / float32
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || (y_dt != MOE_F32 && y_dt != MOE_BF16) ||
        (out_dt != MOE_F32 && out_dt != MOE_BF16))
        return MOE_ERR_INVALID;
    if (K > kMaxCombineK)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!row_of || !out || (y_rows > 0 && !y))
        return MOE_ERR_INVALID;
    if (T > 0x7fffffff || H * ((y_dt == MOE_F32 || out_dt == MOE_F32) ? 4 : 2) > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    if (y_dt == MOE_BF16)
        return out_dt == MOE_BF16 ? launch_combine<uint16_t, uint16_t>(y, y_rows, H, row_of, w, bias, T, K, out, stream)
                                  : launch_combine<uint16_t, float>(y, y_rows, H, row_of, w, bias, T, K, out, stream);
    return out_dt == MOE_BF16 ? launch_combine<float, uint16_t>(y, y_rows, H, row_of, w, bias, T, K, out, stream)
                              : launch_combine<float, float>(y, y_rows, H, row_of, w, bias, T, K, out, stream);
}

extern "C" moe_status moe_group_precombine(const void *y, moe_dtype y_dt, int64_t y_rows, int64_t H,
                                           const int32_t *row_of, const float *w, const int32_t *topk_idx,
                                           int64_t T, int32_t K, int32_t E, int32_t group_size,
                                           const int32_t *slot_of, int64_t slots_cap, void *partials,
                                           moe_dtype partials_dt, hipStream_t stream)
{
    using namespace moe;
    if (y_dt == MOE_FP8_E4M3 || partials_dt == MOE_FP8_E4M3)
        return MOE_ERR_UNSUPPORTED;
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || E < 1 || group_size < 1 || E % group_size != 0 ||
        slots_cap < 0 || (y_dt != MOE_F32 && y_dt != MOE_BF16) || (partials_dt != MOE_F32 && partials_dt != MOE_BF16))
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!row_of || !topk_idx || !slot_of || (slots_cap > 0 && !partials) || (y_rows > 0 && !y))
        return MOE_ERR_INVALID;
    if (T > 0x7fffffff || H * 4 > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    if (y_dt == MOE_BF16)
        return partials_dt == MOE_BF16
                   ? launch_precombine<uint16_t, uint16_t>(y, y_rows, H, row_of, w, topk_idx, T, K, E, group_size,
                                                           slot_of, slots_cap, partials, stream)
                   : launch_precombine<uint16_t, float>(y, y_rows, H, row_of, w, topk_idx, T, K, E, group_size,
                                                        slot_of, slots_cap, partials, stream);
    return partials_dt == MOE_BF16
               ? launch_precombine<float, uint16_t>(y, y_rows, H, row_of, w, topk_idx, T, K, E, group_size, slot_of,
                                                    slots_cap, partials, stream)
               : launch_precombine<float, float>(y, y_rows, H, row_of, w, topk_idx, T, K, E, group_size, slot_of,
                                                 slots_cap, partials, stream);
}

extern "C" moe_status moe_unpermute_combine_backward(const void *dout, moe_dtype dout_dt, const void *y, moe_dtype y_dt,
                                                     int64_t y_rows, int64_t H, const int32_t *row_of, const float *w,
                                                     int64_t T, int32_t K, const int32_t *src_row, void *dy,
                                                     moe_dtype dy_dt, float *dw, hipStream_t stream)
{
    using namespace moe;
    auto dt_ok = [](moe_dtype d) { return d == MOE_F32 || d == MOE_BF16; };
    if (dout_dt == MOE_FP8_E4M3 || y_dt == MOE_FP8_E4M3 || dy_dt == MOE_FP8_E4M3)
        return MOE_ERR_UNSUPPORTED;
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || !dt_ok(dout_dt) || !dt_ok(y_dt) || !dt_ok(dy_dt))
        return MOE_ERR_INVALID;
    if (K > kMaxCombineK)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0 && (y_rows == 0 || !src_row))
        return MOE_OK;
    if ((T > 0 && (!row_of || !dout)) || (y_rows > 0 && !dy) || (dw && y_rows > 0 && !y))
        return MOE_ERR_INVALID;
    if (T > 0x7fffffff || H * 4 > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    if (dout_dt == MOE_BF16)
        return y_dt == MOE_BF16
                   ? launch_combine_backward_dy<uint16_t, uint16_t>(dy_dt, dout, y, y_rows, H, row_of, w, T, K, src_row, dy,
                                                                    dw, stream)
                   : launch_combine_backward_dy<uint16_t, float>(dy_dt, dout, y, y_rows, H, row_of, w, T, K, src_row, dy,
                                                                 dw, stream);
    return y_dt == MOE_BF16
               ? launch_combine_backward_dy<float, uint16_t>(dy_dt, dout, y, y_rows, H, row_of, w, T, K, src_row, dy, dw,
                                                             stream)
               : launch_combine_backward_dy<float, float>(dy_dt, dout, y, y_rows, H, row_of, w, T, K, src_row, dy, dw,
                                                          stream);
}
