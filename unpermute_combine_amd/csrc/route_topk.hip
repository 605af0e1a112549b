// Top-k routing with a softmax over the selected logits, [Scratch] §3 / §27
// ("从零理解 MoE 算子：路由、专家并行与 Token 重排"): topk over router_logits, then softmax of the
// K selected scores.
//
// One wavefront per token. Lane l holds the logits of experts l, l+64, l+128, ... as 64-bit
// keys (order-preserving image of the float in the high word, ~id in the low word), so that
// one unsigned max picks the larger logit and, on a tie, the lower id. Each of the K rounds is
// a wave-wide max (shuffle butterfly); only the winning lane rescans its own keys. The softmax
// runs in double on lanes 0..K-1 and sums in slot order.
#include "moe_common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t score_key(float s, int e)
{
    if (s == 0.0f)
        s = 0.0f;  // -0 and +0 compare equal: same key, so the lower id wins
    uint32_t u = __float_as_uint(s);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_score(uint64_t key)
{
    uint32_t u = static_cast<uint32_t>(key >> 32);
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(u);
}

__device__ __forceinline__ int key_id(uint64_t key)
{
    return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
        uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
        uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

template <int NJ>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int64_t T,
                                                         int E, int K, int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_w)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T)
        return;  // uniform per wave
    const float *row = logits + t * E;

    uint64_t key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + j * kWave;
        key[j] = e < E ? score_key(row[e], e) : 0ull;  // 0 is below every real key
    }
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        best = key[j] > best ? key[j] : best;

    uint64_t mine = 0;  // lane k keeps the key of slot k
    float s0 = 0.0f;
    for (int k = 0; k < K; ++k) {
        const uint64_t win = wave_max_u64(best);
        if (k == 0)
            s0 = key_score(win);
        if (lane == k)
            mine = win;
        if (best == win) {  // exactly one lane: ids are unique
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                key[j] = key[j] == win ? 0ull : key[j];
            best = 0;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                best = key[j] > best ? key[j] : best;
        }
    }

    const bool has = lane < K;
    double ex = has ? exp(static_cast<double>(key_score(mine)) - static_cast<double>(s0)) : 0.0;
    double z = 0.0;
    for (int k = 0; k < K; ++k) {
        const uint32_t lo = __shfl(static_cast<uint32_t>(__double_as_longlong(ex)), k, kWave);
        const uint32_t hi = __shfl(static_cast<uint32_t>(__double_as_longlong(ex) >> 32), k, kWave);
        z += __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
    }
    if (has) {
        topk_idx[t * K + lane] = key_id(mine);
        topk_w[t * K + lane] = static_cast<float>(ex / z);
    }
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_route_topk(const float *logits, int64_t T, int32_t E, int32_t K,
                                     int32_t *topk_idx, float *topk_w, hipStream_t stream)
{
    using namespace moe;
    if (T < 0 || E < 1 || K < 1 || K > E)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!logits || !topk_idx || !topk_w)
        return MOE_ERR_INVALID;
    constexpr int kThreads = 256;
    constexpr int kTokensPerBlock = kThreads / kWave;
    const int64_t blocks = ceil_div(T, kTokensPerBlock);
    if (blocks > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    const int nj = static_cast<int>(ceil_div(E, kWave));
    if (nj <= 1)
        hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, stream, logits, T, E, K, topk_idx, topk_w);
    else if (nj <= 2)
        hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, stream, logits, T, E, K, topk_idx, topk_w);
    else if (nj <= 4)
        hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, stream, logits, T, E, K, topk_idx, topk_w);
    else if (nj <= 8)
        hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, stream, logits, T, E, K, topk_idx, topk_w);
    else
        hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, stream, logits, T, E, K, topk_idx, topk_w);
    return launch_status();
}
