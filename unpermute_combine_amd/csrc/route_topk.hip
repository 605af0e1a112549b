// Top-k routing with a softmax over the selected logits, [Scratch] §3 / §27
// ("从零理解 MoE 算子：路由、专家并行与 Token 重排"): topk over router_logits, then softmax of the
// K selected scores.
//
// gfx950 design: 16 lanes per token, 4 tokens per wavefront. Lane l of a token's 16-lane row
// holds the logits of experts l, l+16, l+32, ... and keeps the best of its own still-unselected
// experts. (Consecutive experts per lane, with 16-byte loads, took 17.7 us instead of 12.7 us at
// T16384 E256 K8 with Zipf-skewed logits: the popular low ids then sit in one or two lanes,
// whose candidate caches run dry.) A key is the logit's order-preserving 32-bit image (-0 taken
// as +0); among equal keys the lower expert id comes first. Each lane keeps its best three keys
// in order (key descending, id ascending). Each of the K rounds takes the maximum of the lanes'
// first keys over the 16 lanes with four DPP max steps (row_mirror, row_half_mirror, quad xor 2,
// quad xor 1: VALU instructions, no LDS round trip); the lanes holding that key are the
// candidates, found with one ballot, and only when a row has two candidates (equal logits) does a
// second 16-lane DPP reduction pick the lowest expert id among them. The winner lane records the
// slot in LDS and moves its next keys up; it rescans its keys only once all three are gone.
// Measured at T16384 E256 K8 (event time per launch): 15.4 us with a (key, ~id) pair reduced
// each round and one load wait per key, 13.3 us with the loads in flight together, 12.0 us with
// the keys-only max. The softmax runs in double; the K exponentials meet in LDS and every lane
// sums them in slot order.
//
// Group-limited routing ([Scratch] §21: pick a few expert groups first, then the experts inside
// them) runs in the same kernel before the K rounds: the lanes fold their keys into per-group
// maxima with LDS atomic max (on the order-preserving keys, so the maximum key is the group's
// best logit), then topk_groups rounds of a 16-lane DPP reduction of (group key, ~group id)
// pairs pick the groups, and the experts of the other groups are dropped from the candidates.
// That code lives only in the group-limited instance (GROUPS), and the candidate refill is inlined
// once: with caches flushed the kernel's code is fetched from HBM as it runs, and the plain
// E = 256 kernel shrank from 15.9 to 6.5 KB (9.2 -> 8.9 us at T16384 K8, 6.8 -> 6.6 us at T8192).
#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kLanesPerToken = 16;
constexpr int kRouteThreads = 256;
constexpr int kTokensPerBlock = kRouteThreads / kLanesPerToken;  // 16
constexpr int kSlotRegs = (MOE_MAX_TOPK + kLanesPerToken - 1) / kLanesPerToken;  // slots per lane

// DPP controls (gfx9 encoding)
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xb1;  // quad_perm [1,0,3,2]

__device__ __forceinline__ uint32_t orderable(float s)
{
    if (s == 0.0f)
        s = 0.0f;  // -0 and +0 compare equal: same key, so the lower id wins
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // > 0 for every non-NaN float
}

__device__ __forceinline__ float from_orderable(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ void max_step(uint32_t &hi, uint32_t &lo)
{
    const uint32_t ohi = dpp<CTRL>(hi);
    const uint32_t olo = dpp<CTRL>(lo);
    const bool gt = ohi > hi || (ohi == hi && olo > lo);
    hi = gt ? ohi : hi;
    lo = gt ? olo : lo;
}

// Largest (hi, lo) of the 16 lanes of this lane's row, in every lane of the row.
__device__ __forceinline__ void row_max(uint32_t &hi, uint32_t &lo)
{
    max_step<kDppRowMirror>(hi, lo);
    max_step<kDppRowHalfMirror>(hi, lo);
    max_step<kDppQuadXor2>(hi, lo);
    max_step<kDppQuadXor1>(hi, lo);
}

// Largest (or smallest) of one 32-bit value over the 16 lanes of this lane's row.
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v)
{
    return max(v, dpp<CTRL>(v));
}

template <int CTRL>
__device__ __forceinline__ uint32_t min_dpp(uint32_t v)
{
    return min(v, dpp<CTRL>(v));
}

__device__ __forceinline__ uint32_t row_max1(uint32_t v)
{
    return max_dpp<kDppQuadXor1>(max_dpp<kDppQuadXor2>(max_dpp<kDppRowHalfMirror>(max_dpp<kDppRowMirror>(v))));
}

__device__ __forceinline__ uint32_t row_min1(uint32_t v)
{
    return min_dpp<kDppQuadXor1>(min_dpp<kDppQuadXor2>(min_dpp<kDppRowHalfMirror>(min_dpp<kDppRowMirror>(v))));
}

constexpr int kMaxRouteGroups = 256;  // group keys in LDS: 16 tokens x 256 x 4 B per workgroup
constexpr uint32_t kChosenGroup = 0xffffffffu;  // above every key of a finite logit

// Per-tile expert (and group) counts of the routed slots, kept in LDS by the fused route + tile
// count kernel: he[e] += 1 for every selected expert, hg[g] += 1 for the first of a token's slots
// in each group of gs experts (gs = 0: no groups). Counts only, never positions.
struct TileCounts {
    int32_t *he, *hg;
    int gs;
};

// One pass of the routing over the TPB tokens t_first .. t_first + TPB - 1 of this workgroup
// (16 lanes per token; tokens at or past t_end take part with empty keys and store nothing).
// HIST: the selected experts are also counted into `tc`.
template <int J, bool GROUPS, int TPB, bool HIST>
__device__ __forceinline__ void route_pass(const float *__restrict__ logits, int64_t T, int64_t t_first, int64_t t_end,
                                           int E, int K, int gs, int M, int32_t *__restrict__ topk_idx,
                                           float *__restrict__ topk_w, TileCounts tc)
{
    __shared__ double ex_sh[TPB][MOE_MAX_TOPK];
    extern __shared__ uint32_t group_sh[];  // [TPB][G] when gs > 0
    const int sub = threadIdx.x & (kLanesPerToken - 1);
    const int tok = threadIdx.x / kLanesPerToken;  // token of this row inside the block
    const int64_t t = t_first + tok;
    const bool live = t < t_end;  // rows past the end take part in the DPP steps with empty keys
    // every load in bounds (rows past T read row T-1, experts past E read expert E-1) and the
    // absent ones masked afterwards: the J loads issue back to back with one wait (a guarded
    // load per key made the compiler wait for each one before issuing the next: 15.4 against
    // 13.3 us per launch, event time, at T16384 E256 K8; 23.0 against 18.8 us with group-limited
    // routing at T8192 E256)
    const float *row = logits + (live ? t : T - 1) * E;
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = sub + kLanesPerToken * j;
        v[j] = __builtin_nontemporal_load(row + (e < E ? e : E - 1));
    }
    uint32_t u[J];  // orderable logits of experts sub + 16 j; 0 = absent or already selected
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int e = sub + kLanesPerToken * j;
        u[j] = (live && e < E) ? orderable(v[j]) : 0u;
    }
    if (GROUPS) {  // group-limited: keep only the experts of the M best groups
        const int G = E / gs;
        uint32_t *gk = group_sh + tok * G;
        for (int g = sub; g < G; g += kLanesPerToken)
            gk[g] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (u[j])
                atomicMax(&gk[(sub + kLanesPerToken * j) / gs], u[j]);
        __syncthreads();
        uint32_t gu[J];  // keys of groups sub + 16 q (G <= E, so J registers suffice)
        uint32_t gbu = 0;
        int gbq = 0;
#pragma unroll
        for (int q = 0; q < J; ++q) {
            const int g = sub + kLanesPerToken * q;
            gu[q] = g < G ? gk[g] : 0u;
            if (gu[q] > gbu) {
                gbu = gu[q];
                gbq = q;
            }
        }
        for (int m = 0; m < M; ++m) {
            uint32_t hi = gbu;
            uint32_t lo = gbu ? 0xffffffffu - static_cast<uint32_t>(sub + kLanesPerToken * gbq) : 0u;
            row_max(hi, lo);
            const int wg = static_cast<int>(0xffffffffu - lo);  // winning group of this row
            if (hi != 0 && sub == (wg & (kLanesPerToken - 1))) {
                const int wq = wg / kLanesPerToken;
                gbu = 0;
                gbq = 0;
#pragma unroll
                for (int q = 0; q < J; ++q) {
                    if (q == wq)
                        gu[q] = 0;
                    if (gu[q] > gbu) {
                        gbu = gu[q];
                        gbq = q;
                    }
                }
            }
            if (hi != 0 && sub == 0)
                gk[wg] = kChosenGroup;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (u[j] && gk[(sub + kLanesPerToken * j) / gs] != kChosenGroup)
                u[j] = 0;
    }

    // This lane's candidates: the best three of its keys not yet given up, in order (key
    // descending, then expert id ascending). Each round the 16 lanes of a token compare their
    // first candidates; the winner's owner drops it and moves the next ones up, and only a
    // lane that has given up all three of a full cache rescans its keys (`taken` marks what it
    // gave up). Scanning j upwards with strict > keeps the lowest id first among equal keys.
    uint32_t cu0 = 0, cu1 = 0, cu2 = 0;
    int cj0 = 0, cj1 = 0, cj2 = 0;
    uint64_t taken = 0;
    auto fill = [&]() {
        cu0 = cu1 = cu2 = 0;
        cj0 = cj1 = cj2 = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint32_t x = ((taken >> j) & 1u) ? 0u : u[j];
            const bool g0 = x > cu0, g1 = x > cu1, g2 = x > cu2;
            cu2 = g1 ? cu1 : (g2 ? x : cu2);
            cj2 = g1 ? cj1 : (g2 ? j : cj2);
            cu1 = g0 ? cu0 : (g1 ? x : cu1);
            cj1 = g0 ? cj0 : (g1 ? j : cj1);
            cu0 = g0 ? x : cu0;
            cj0 = g0 ? j : cj0;
        }
    };
    bool complete = false;  // fewer than three keys: the cache holds all that are left

    // Each round: the token's largest first key (a 16-lane max of the keys alone); the lanes
    // holding it are the candidates, and only when two candidates hold equal keys does a
    // second 16-lane reduction pick the lowest expert id among them. The winner lane records
    // the slot in LDS and gives up its first key.
    __shared__ uint32_t slot_key[TPB][MOE_MAX_TOPK];
    __shared__ int32_t slot_id[TPB][MOE_MAX_TOPK];
    const int seg_shift = threadIdx.x & (kWave - kLanesPerToken);  // this row's first lane in the wave
    uint32_t s0u = 0;
    for (int k = 0; k < K; ++k) {
        if (cu0 == 0 && !complete) {  // (re)fill the cache: the first round, and after giving up three
            fill();
            complete = cu2 == 0;
        }
        const uint32_t m = row_max1(cu0);
        if (k == 0)
            s0u = m;
        const bool cand = cu0 != 0 && cu0 == m;
        const uint32_t seg = static_cast<uint32_t>(__ballot(cand) >> seg_shift) & ((1u << kLanesPerToken) - 1);
        bool win = cand;
        if (__ballot(__popc(seg) > 1)) {  // equal keys in some row: the lowest expert id wins
            const uint32_t id = cand ? static_cast<uint32_t>(sub + kLanesPerToken * cj0) : 0xffffffffu;
            const uint32_t lowest = row_min1(id);  // every lane of the wavefront takes part
            win = cand && id == lowest;
        }
        if (win) {
            slot_key[tok][k] = cu0;
            slot_id[tok][k] = sub + kLanesPerToken * cj0;
            taken |= 1ull << cj0;
            cu0 = cu1;
            cj0 = cj1;
            cu1 = cu2;
            cj1 = cj2;
            cu2 = 0;
        }
    }
    __builtin_amdgcn_wave_barrier();

    // softmax over the K selected logits, in double, summed in slot order
    const double s0 = static_cast<double>(from_orderable(s0u));
    double ex[kSlotRegs];
    int32_t slot_e[kSlotRegs];
#pragma unroll
    for (int q = 0; q < kSlotRegs; ++q) {
        const int k = sub + kLanesPerToken * q;
        ex[q] = 0.0;
        slot_e[q] = 0;
        if (k < K) {
            ex[q] = exp(static_cast<double>(from_orderable(slot_key[tok][k])) - s0);
            slot_e[q] = slot_id[tok][k];
            ex_sh[tok][k] = ex[q];
        }
    }
    __builtin_amdgcn_wave_barrier();
    double z = 0.0;
    for (int k = 0; k < K; ++k)
        z += ex_sh[tok][k];
    if (live) {
#pragma unroll
        for (int q = 0; q < kSlotRegs; ++q) {
            const int k = sub + kLanesPerToken * q;
            if (k < K) {
                topk_idx[t * K + k] = slot_e[q];
                topk_w[t * K + k] = static_cast<float>(ex[q] / z);
                if constexpr (HIST) {
                    const int e = slot_e[q];
                    atomicAdd(&tc.he[e], 1);
                    if (tc.gs > 0) {  // the token's first slot in its group
                        const int g = e / tc.gs;
                        bool lead = true;
                        for (int j = 0; j < k; ++j)
                            lead = lead && slot_id[tok][j] / tc.gs != g;
                        if (lead)
                            atomicAdd(&tc.hg[g], 1);
                    }
                }
            }
        }
    }
}

template <int J, bool GROUPS>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(const float *__restrict__ logits, int64_t T,
                                                                   int E, int K, int gs, int M,
                                                                   int32_t *__restrict__ topk_idx,
                                                                   float *__restrict__ topk_w)
{
    route_pass<J, GROUPS, kTokensPerBlock, false>(logits, T, static_cast<int64_t>(blockIdx.x) * kTokensPerBlock, T, E,
                                                  K, gs, M, topk_idx, topk_w, TileCounts{});
}

// ---------------------------------------------------------------- fused route + tile counts
// The routing of moe_route_topk_index for inputs whose index build counts tiles ([Scratch] §3:
// top-k and softmax; §7: the per-expert counts behind group_list): one workgroup per index tile
// of whole tokens, 64 tokens per pass, so that the workgroup that routes a tile also counts its
// slots -- per expert, and with index groups per (token, group) first slot -- into one row of
// tile counts, the rows the rank pass of the index build reads. This replaces the separate
// histogram launch, which re-read topk_idx.
constexpr int kFusedTokens = 64;
constexpr int kFusedThreads = kFusedTokens * kLanesPerToken;  // 1024
constexpr int kFusedMaxTiles = 256;

struct CountArgs {
    int32_t tile_tokens;
    int32_t idx_gs, G;  // index groups (idx_gs = 0: none)
    int32_t Ep, Hp;     // E and G rounded up to multiples of 4; Hp = Ep (+ Gp): a tile's row
    int32_t *hist;      // [tiles][Hp]
    int32_t *slot_of;   // [T][G]: -1 for the tile's tokens (index group mode)
};

template <int J>
__global__ __launch_bounds__(kFusedThreads) void route_count_kernel(const float *__restrict__ logits, int64_t T, int E,
                                                                    int K, int32_t *__restrict__ topk_idx,
                                                                    float *__restrict__ topk_w, CountArgs c)
{
    extern __shared__ int32_t cnt[];  // the tile's row of counts
    for (int i = threadIdx.x; i < c.Hp; i += kFusedThreads)
        cnt[i] = 0;
    __syncthreads();
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * c.tile_tokens;
    const int64_t t1 = min(T, t0 + c.tile_tokens);
    const TileCounts tc{cnt, cnt + c.Ep, c.idx_gs};
    for (int64_t tf = t0; tf < t1; tf += kFusedTokens)
        route_pass<J, false, kFusedTokens, true>(logits, T, tf, t1, E, K, 0, 0, topk_idx, topk_w, tc);
    if (c.idx_gs > 0) {  // slot_of starts as "absent" for this tile's tokens
        for (int64_t i = t0 * c.G + threadIdx.x; i < t1 * c.G; i += kFusedThreads)
            c.slot_of[i] = -1;
    }
    __syncthreads();
    int32_t *row = c.hist + static_cast<int64_t>(blockIdx.x) * c.Hp;
    for (int i = threadIdx.x; i < c.Hp; i += kFusedThreads)
        row[i] = cnt[i];
}

// ---------------------------------------------------------------- backward
// Gradient of the logits through the softmax over the K selected logits ([Scratch] §3/§27: the
// softmax runs over the selected scores; [Combine] §6: only the selected experts carry router
// gradient, the selection itself being piecewise constant). With w = topk_w and g = d_topk_w:
//   d_logits[t, topk_idx[t,k]] += w[t,k] * (g[t,k] - sum_j w[t,j] g[t,j])
// in double -- the sum over j in slot order, the slots in order -- rounded once to float32; every
// other logit gets 0. One wavefront per token: lanes 0..K-1 hold the slots, every lane forms the
// same sum from them with readlane, and each lane writes whole positions of the row (no two
// lanes write one entry).
constexpr int kBwdTokensPerBlock = kRouteThreads / kWave;

__global__ __launch_bounds__(kRouteThreads) void route_topk_backward_kernel(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, const float *__restrict__ d_topk_w, int64_t T,
    int E, int K, float *__restrict__ d_logits)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kBwdTokensPerBlock +
                      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    if (t >= T)
        return;
    const bool mine = lane < K;
    const int32_t id = mine ? topk_idx[t * K + lane] : -1;
    const float wk = mine ? topk_w[t * K + lane] : 0.0f;
    const float gk = mine ? d_topk_w[t * K + lane] : 0.0f;
    double s = 0.0;
    for (int j = 0; j < K; ++j)
        s += static_cast<double>(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), j))) *
             static_cast<double>(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(gk), j)));
    for (int e = lane; e < E; e += kWave) {
        double v = 0.0;
        for (int k = 0; k < K; ++k) {
            if (__builtin_amdgcn_readlane(id, k) != e)
                continue;
            const double w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), k));
            const double g1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gk), k));
            v += w1 * (g1 - s);
        }
        d_logits[t * E + e] = static_cast<float>(v);
    }
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {

moe_status launch_route(const float *logits, int64_t T, int32_t E, int32_t K, int32_t gs, int32_t M,
                        int32_t *topk_idx, float *topk_w, hipStream_t stream)
{
    if (T == 0)
        return MOE_OK;
    if (!logits || !topk_idx || !topk_w)
        return MOE_ERR_INVALID;
    const int64_t blocks = ceil_div(T, kTokensPerBlock);
    if (blocks > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kRouteThreads);
    const size_t lds = gs > 0 ? sizeof(uint32_t) * kTokensPerBlock * static_cast<size_t>(E / gs) : 0;
    const int nj = static_cast<int>(ceil_div(E, kLanesPerToken));
#define MOE_ROUTE_LAUNCH(JJ) \
    do {                                                                                                         \
        if (gs > 0)                                                                                              \
            hipLaunchKernelGGL((route_topk_kernel<JJ, true>), grid, block, lds, stream, logits, T, E, K, gs, M,      \
                               topk_idx, topk_w);                                                                \
        else                                                                                                     \
            hipLaunchKernelGGL((route_topk_kernel<JJ, false>), grid, block, lds, stream, logits, T, E, K, gs, M,     \
                               topk_idx, topk_w);                                                                \
    } while (0)
    if (nj <= 1)
        MOE_ROUTE_LAUNCH(1);
    else if (nj <= 2)
        MOE_ROUTE_LAUNCH(2);
    else if (nj <= 4)
        MOE_ROUTE_LAUNCH(4);
    else if (nj <= 8)
        MOE_ROUTE_LAUNCH(8);
    else if (nj <= 16)
        MOE_ROUTE_LAUNCH(16);
    else if (nj <= 32)
        MOE_ROUTE_LAUNCH(32);
    else
        MOE_ROUTE_LAUNCH(64);
#undef MOE_ROUTE_LAUNCH
    return launch_status();
}

// The fused route when the index build counts tiles, E <= 256 and the routing is not
// group-limited: with 1024-thread workgroups a thread has 128 registers, and the routing of more
// experts per lane, or the group-limited routing, spills (J = 32: 75 to 112 registers to scratch;
// group-limited at E = 256: 28 us against 13 + 5 us for the separate route and histogram).
// Otherwise moe_route_topk_index makes the two separate calls.
bool use_fused(int64_t T, int32_t K, int32_t E, int32_t route_group_size)
{
    return build_index_counts_tiles(T, K) && ceil_div(E, kLanesPerToken) <= 16 && route_group_size <= 0;
}

// Tiles of the fused route: a multiple of its 64-token passes, at most kFusedMaxTiles of them.
int32_t fused_tile_tokens(int64_t T)
{
    const int64_t tt = ceil_div(ceil_div(T, kFusedMaxTiles), kFusedTokens) * kFusedTokens;
    return static_cast<int32_t>(tt < kFusedTokens ? kFusedTokens : tt);
}

// Bytes of the tile counts the fused route writes (the rank pass's rows; 256-byte rounded).
size_t fused_counts_bytes(int64_t T, int32_t E, int32_t group_size)
{
    const int64_t ntiles = ceil_div(T, fused_tile_tokens(T));
    const int64_t hp = ((E + 3) & ~3) + (group_size > 0 ? ((E / group_size + 3) & ~3) : 0);
    const size_t b = sizeof(int32_t) * static_cast<size_t>(hp * ntiles);
    return (b + 255) & ~static_cast<size_t>(255);
}

moe_status check_route(int64_t T, int32_t E, int32_t K, int32_t gs, int32_t M)
{
    if (T < 0 || E < 1 || K < 1 || K > E)
        return MOE_ERR_INVALID;
    if (gs > 0 && (E % gs != 0 || M < 1 || M > E / gs || static_cast<int64_t>(K) > static_cast<int64_t>(M) * gs))
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK || (gs > 0 && E / gs > kMaxRouteGroups))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status launch_route_count(const float *logits, int64_t T, int32_t E, int32_t K, int32_t *topk_idx, float *topk_w,
                              const CountArgs &c, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(ceil_div(T, c.tile_tokens))), block(kFusedThreads);
    const size_t lds = sizeof(int32_t) * static_cast<size_t>(c.Hp);
    const int nj = static_cast<int>(ceil_div(E, kLanesPerToken));
#define MOE_ROUTE_COUNT_LAUNCH(JJ)                                                                                   \
    hipLaunchKernelGGL((route_count_kernel<JJ>), grid, block, lds, stream, logits, T, E, K, topk_idx, topk_w, c)
    if (nj <= 1)
        MOE_ROUTE_COUNT_LAUNCH(1);
    else if (nj <= 2)
        MOE_ROUTE_COUNT_LAUNCH(2);
    else if (nj <= 4)
        MOE_ROUTE_COUNT_LAUNCH(4);
    else if (nj <= 8)
        MOE_ROUTE_COUNT_LAUNCH(8);
    else if (nj <= 16)
        MOE_ROUTE_COUNT_LAUNCH(16);
    else
        return MOE_ERR_UNSUPPORTED;  // more than 256 experts take the separate calls (use_fused)
#undef MOE_ROUTE_COUNT_LAUNCH
    return launch_status();
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
    return launch_route(logits, T, E, K, 0, 0, topk_idx, topk_w, stream);
}

extern "C" moe_status moe_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t K,
                                             int32_t group_size, int32_t topk_groups, int32_t *topk_idx,
                                             float *topk_w, hipStream_t stream)
{
    using namespace moe;
    if (T < 0 || E < 1 || K < 1 || K > E || group_size < 1 || E % group_size != 0 || topk_groups < 1 ||
        topk_groups > E / group_size || static_cast<int64_t>(K) > static_cast<int64_t>(topk_groups) * group_size)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK || E / group_size > kMaxRouteGroups)
        return MOE_ERR_UNSUPPORTED;
    return launch_route(logits, T, E, K, group_size, topk_groups, topk_idx, topk_w, stream);
}

extern "C" moe_status moe_route_topk_backward(const int32_t *topk_idx, const float *topk_w, const float *d_topk_w,
                                              int64_t T, int32_t E, int32_t K, float *d_logits, hipStream_t stream)
{
    using namespace moe;
    if (T < 0 || E < 1 || K < 1 || K > E)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!topk_idx || !topk_w || !d_topk_w || !d_logits)
        return MOE_ERR_INVALID;
    const int64_t blocks = ceil_div(T, kBwdTokensPerBlock);
    if (blocks > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(route_topk_backward_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kRouteThreads), 0, stream,
                       topk_idx, topk_w, d_topk_w, T, E, K, d_logits);
    return launch_status();
}

extern "C" moe_status moe_route_topk_index_workspace_size(int64_t T, int32_t K, int32_t E, int32_t group_size,
                                                          size_t *bytes)
{
    using namespace moe;
    if (!bytes)
        return MOE_ERR_INVALID;
    size_t separate = 0;
    const moe_status st = moe_build_index_workspace_size(T, K, E, group_size, &separate);
    if (st != MOE_OK)
        return st;
    // enough for either path (the fused one has at least as many tiles)
    *bytes = use_fused(T, K, E, 0) ? std::max(fused_counts_bytes(T, E, group_size), separate) : separate;
    return MOE_OK;
}

extern "C" moe_status moe_route_topk_index(const float *logits, int64_t T, int32_t E, int32_t K,
                                           int32_t route_group_size, int32_t topk_groups, int32_t *topk_idx,
                                           float *topk_w, int32_t capacity, int32_t group_size, int32_t alignment,
                                           const moe_index *out, void *workspace, size_t workspace_bytes,
                                           hipStream_t stream)
{
    using namespace moe;
    const int32_t rgs = route_group_size > 0 ? route_group_size : 0;
    moe_status st = check_route(T, E, K, rgs, rgs > 0 ? topk_groups : 0);
    if (st != MOE_OK)
        return st;
    // every index argument error before any launch
    st = build_index_from_tile_counts(topk_idx, topk_w, T, K, E, capacity, group_size, alignment, out, nullptr, 0,
                                      fused_tile_tokens(T), false, stream);
    if (st != MOE_OK)
        return st;
    if (T > 0 && (!logits || !topk_idx || !topk_w))
        return MOE_ERR_INVALID;
    size_t need = 0;
    if ((st = moe_route_topk_index_workspace_size(T, K, E, group_size, &need)) != MOE_OK)
        return st;
    if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace))))
        return MOE_ERR_INVALID;
    if (!use_fused(T, K, E, rgs)) {  // the two calls
        if ((st = launch_route(logits, T, E, K, rgs, topk_groups, topk_idx, topk_w, stream)) != MOE_OK)
            return st;
        return moe_build_index(topk_idx, topk_w, T, K, E, capacity, group_size, alignment, out, workspace,
                               workspace_bytes, stream);
    }
    CountArgs c{};
    c.tile_tokens = fused_tile_tokens(T);
    c.idx_gs = group_size > 0 ? group_size : 0;
    c.G = group_size > 0 ? E / group_size : 0;
    c.Ep = (E + 3) & ~3;
    c.Hp = c.Ep + (c.G > 0 ? ((c.G + 3) & ~3) : 0);
    c.hist = static_cast<int32_t *>(workspace);
    c.slot_of = out->slot_of;
    if ((st = launch_route_count(logits, T, E, K, topk_idx, topk_w, c, stream)) != MOE_OK)
        return st;
    return build_index_from_tile_counts(topk_idx, topk_w, T, K, E, capacity, group_size, alignment, out, workspace,
                                        workspace_bytes, c.tile_tokens, true, stream);
}
