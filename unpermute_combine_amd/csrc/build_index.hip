// Expert-major index build: a stable counting sort of the T*K routing slots by expert.
//
// Definition followed ([Megatron] §1.1, "token dispatcher + fuse_a2a", permute()): the routing
// map is transposed to [experts, tokens] and masked_select lists, expert by expert, the tokens
// routed there in ascending order -> sorted_indices; the same mask over the transposed probs
// gives permuted_probs; [Scratch] §7 ("从零理解 MoE 算子") gives group_list as the running sum
// of the per-expert counts. Ordering the slots i = t*K + k by (expert, i) is exactly that list.
//
// gfx950 design (three launches, plus one in group mode):
//   1. hist   one workgroup per tile of whole tokens: per-tile expert histogram (and group
//             histogram of the first slot of each (token, group)) with LDS atomics -- only the
//             counts, never positions, come from atomics, so the result is deterministic.
//   2. scan   one workgroup: exclusive scan of the [key][tile] histograms in key-major order,
//             giving every (key, tile) its first row; counts, group_list, capacity bookkeeping,
//             padding and unused rows.
//   3. rank   one wavefront per tile walks its slots 64 at a time in slot order. Lanes with
//             the same key find each other with one ballot per key bit (a match-any built from
//             ballots), their stable rank is popcount(peers & lanes_below), and the last peer
//             advances the key's running row counter in LDS.
//   4. esrc   (group mode) expert-major row -> group slot.
// The drop-and-pad capacity rule ([Scratch] §18, §26.6) and the group (send once per rank)
// slots ([CANN] §1(1)) are applied inside the same passes.
#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

struct IndexArgs {
    const int32_t *topk_idx;
    const float *topk_w;
    int64_t T;
    int32_t K, E, cap, gs, G;
    int32_t tile_tokens, ntiles;
    int32_t ebits, gbits;
    int32_t *hist_e;  // [E][ntiles] -> exclusive bases after the scan
    int32_t *hist_g;  // [G][ntiles]
    moe_index ix;
};

__device__ __forceinline__ bool valid_expert(int e, int E) { return e >= 0 && e < E; }

// True if slot k of a token is the first of that token's slots in expert group g.
__device__ __forceinline__ bool group_leader(const int32_t *ids, int k, int g, int E, int gs)
{
    for (int j = 0; j < k; ++j) {
        const int e = ids[j];
        if (valid_expert(e, E) && e / gs == g)
            return false;
    }
    return true;
}

__global__ __launch_bounds__(256) void hist_kernel(IndexArgs a)
{
    extern __shared__ int32_t sh[];
    int32_t *he = sh;
    int32_t *hg = sh + a.E;
    const int tile = blockIdx.x;
    for (int i = threadIdx.x; i < a.E + (a.gs > 0 ? a.G : 0); i += blockDim.x)
        sh[i] = 0;
    __syncthreads();
    const int64_t t0 = static_cast<int64_t>(tile) * a.tile_tokens;
    const int64_t t1 = min(a.T, t0 + a.tile_tokens);
    const int64_t s0 = t0 * a.K, s1 = t1 * a.K;
    for (int64_t i = s0 + threadIdx.x; i < s1; i += blockDim.x) {
        const int e = a.topk_idx[i];
        if (!valid_expert(e, a.E))
            continue;
        atomicAdd(&he[e], 1);
        if (a.gs > 0) {
            const int64_t t = i / a.K;
            const int k = static_cast<int>(i - t * a.K);
            const int g = e / a.gs;
            if (group_leader(a.topk_idx + t * a.K, k, g, a.E, a.gs))
                atomicAdd(&hg[g], 1);
        }
    }
    if (a.gs > 0) {  // slot_of starts as "absent" for this tile's tokens
        for (int64_t i = t0 * a.G + threadIdx.x; i < t1 * a.G; i += blockDim.x)
            a.ix.slot_of[i] = -1;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += blockDim.x)
        a.hist_e[static_cast<int64_t>(e) * a.ntiles + tile] = he[e];
    if (a.gs > 0)
        for (int g = threadIdx.x; g < a.G; g += blockDim.x)
            a.hist_g[static_cast<int64_t>(g) * a.ntiles + tile] = hg[g];
}

constexpr int kScanThreads = 1024;

// In-place exclusive scan of n ints by one workgroup; returns the total to every thread.
__device__ int64_t block_exclusive_scan(int32_t *v, int64_t n, int32_t *sh_sums)
{
    const int tid = threadIdx.x;
    const int64_t per = (n + kScanThreads - 1) / kScanThreads;
    const int64_t lo = min(n, tid * per), hi = min(n, lo + per);
    int32_t sum = 0;
    for (int64_t i = lo; i < hi; ++i)
        sum += v[i];
    sh_sums[tid] = sum;
    __syncthreads();
    // Hillis-Steele over the 1024 strip sums
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int32_t add = tid >= off ? sh_sums[tid - off] : 0;
        __syncthreads();
        sh_sums[tid] += add;
        __syncthreads();
    }
    const int32_t total = sh_sums[kScanThreads - 1];
    int32_t run = sh_sums[tid] - sum;  // exclusive prefix of this strip
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t c = v[i];
        v[i] = run;
        run += c;
    }
    __syncthreads();
    return total;
}

// First row of key `key` after the scan (its tile-0 base); `total` past the last key.
__device__ __forceinline__ int32_t key_start(const int32_t *bases, int key, int nkeys, int ntiles,
                                             int32_t total)
{
    if (ntiles == 0)
        return 0;
    return key < nkeys ? bases[static_cast<int64_t>(key) * ntiles] : total;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(IndexArgs a)
{
    __shared__ int32_t sums[kScanThreads];
    const int tid = threadIdx.x;
    const int64_t R = a.cap > 0 ? static_cast<int64_t>(a.E) * a.cap : a.T * a.K;
    const int32_t total = static_cast<int32_t>(
        block_exclusive_scan(a.hist_e, static_cast<int64_t>(a.E) * a.ntiles, sums));
    __threadfence_block();
    for (int e = tid; e < a.E; e += kScanThreads) {
        const int32_t start = key_start(a.hist_e, e, a.E, a.ntiles, total);
        const int32_t end = key_start(a.hist_e, e + 1, a.E, a.ntiles, total);
        const int32_t cnt = end - start;
        a.ix.counts[e] = cnt;
        a.ix.group_list[e] = end;
        if (a.ix.kept_counts)
            a.ix.kept_counts[e] = a.cap > 0 ? min(cnt, a.cap) : cnt;
    }
    if (a.cap > 0) {
        // padding rows of every expert: p >= min(count, cap)
        for (int64_t r = tid; r < R; r += kScanThreads) {
            const int e = static_cast<int>(r / a.cap);
            const int p = static_cast<int>(r - static_cast<int64_t>(e) * a.cap);
            const int32_t start = key_start(a.hist_e, e, a.E, a.ntiles, total);
            const int32_t end = key_start(a.hist_e, e + 1, a.E, a.ntiles, total);
            if (p >= min(end - start, a.cap)) {
                a.ix.sorted_indices[r] = -1;
                if (a.ix.permuted_probs)
                    a.ix.permuted_probs[r] = 0.0f;
            }
        }
    } else {
        // rows after the last routed slot are unused
        for (int64_t r = total + tid; r < R; r += kScanThreads) {
            a.ix.sorted_indices[r] = -1;
            if (a.ix.permuted_probs)
                a.ix.permuted_probs[r] = 0.0f;
            if (a.gs > 0)
                a.ix.esrc[r] = -1;
        }
    }
    if (a.gs > 0) {
        __syncthreads();
        const int32_t m = static_cast<int32_t>(
            block_exclusive_scan(a.hist_g, static_cast<int64_t>(a.G) * a.ntiles, sums));
        for (int g = tid; g < a.G; g += kScanThreads) {
            const int32_t start = key_start(a.hist_g, g, a.G, a.ntiles, m);
            const int32_t end = key_start(a.hist_g, g + 1, a.G, a.ntiles, m);
            a.ix.group_counts[g] = end - start;
        }
        if (tid == 0)
            a.ix.n_slots[0] = m;
    }
}

// Bitwise match-any over the low `bits` bits of key among the lanes in `active`.
__device__ __forceinline__ uint64_t match_peers(int key, int bits, uint64_t active)
{
    uint64_t m = active;
    for (int b = 0; b < bits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = __ballot(bit);
        m &= bit ? ones : ~ones;
    }
    return m;
}

__device__ __forceinline__ int last_lane(uint64_t m) { return 63 - __clzll(m); }

__global__ __launch_bounds__(64) void rank_kernel(IndexArgs a)
{
    extern __shared__ int32_t sh[];
    int32_t *run_e = sh;         // next row of each expert in this tile
    int32_t *run_g = sh + a.E;   // next slot of each group in this tile
    const int tile = blockIdx.x;
    const int lane = threadIdx.x;
    for (int e = lane; e < a.E; e += kWave)
        run_e[e] = a.hist_e[static_cast<int64_t>(e) * a.ntiles + tile];
    if (a.gs > 0)
        for (int g = lane; g < a.G; g += kWave)
            run_g[g] = a.hist_g[static_cast<int64_t>(g) * a.ntiles + tile];
    __syncthreads();

    const int64_t t0 = static_cast<int64_t>(tile) * a.tile_tokens;
    const int64_t t1 = min(a.T, t0 + a.tile_tokens);
    const int64_t s0 = t0 * a.K, s1 = t1 * a.K;
    const uint64_t below = lanemask_lt();
    for (int64_t base = s0; base < s1; base += kWave) {
        const int64_t i = base + lane;
        const bool in = i < s1;
        const int e = in ? a.topk_idx[i] : -1;
        const bool ok = valid_expert(e, a.E);
        const int64_t t = i / a.K;
        const int k = static_cast<int>(i - t * a.K);

        // ---- expert-major row
        const uint64_t pe = match_peers(e, a.ebits, __ballot(ok));
        int32_t row = -1;
        if (ok) {
            const int32_t r = run_e[e] + __popcll(pe & below);
            row = r;
            if (a.cap > 0) {
                const int32_t seg = a.hist_e[static_cast<int64_t>(e) * a.ntiles];  // expert's first row
                const int32_t p = r - seg;
                row = p < a.cap ? e * a.cap + p : -1;
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (ok && lane == last_lane(pe))
            run_e[e] += __popcll(pe);
        if (in)
            a.ix.row_of[i] = row;
        if (row >= 0) {
            a.ix.sorted_indices[row] = static_cast<int32_t>(t);
            if (a.ix.permuted_probs)
                a.ix.permuted_probs[row] = a.topk_w ? a.topk_w[i] : 1.0f;
        }

        // ---- group slots: one per (token, group), listed group by group, tokens ascending
        if (a.gs > 0) {
            const int g = ok ? e / a.gs : -1;
            const bool lead = ok && group_leader(a.topk_idx + t * a.K, k, g, a.E, a.gs);
            const uint64_t pg = match_peers(g, a.gbits, __ballot(lead));
            int32_t slot = -1;
            if (lead)
                slot = run_g[g] + __popcll(pg & below);
            __builtin_amdgcn_wave_barrier();
            if (lead && lane == last_lane(pg))
                run_g[g] += __popcll(pg);
            if (lead) {
                a.ix.slot_of[t * a.G + g] = slot;
                a.ix.gsrc[slot] = static_cast<int32_t>(t);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

__global__ __launch_bounds__(256) void esrc_kernel(IndexArgs a)
{
    const int64_t n = a.T * a.K;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int e = a.topk_idx[i];
        const int32_t row = a.ix.row_of[i];
        if (!valid_expert(e, a.E) || row < 0)
            continue;
        const int64_t t = i / a.K;
        a.ix.esrc[row] = a.ix.slot_of[t * a.G + e / a.gs];
    }
}

int bits_for(int n)  // bits needed to tell apart the keys 0..n-1
{
    int b = 0;
    while ((1 << b) < n)
        ++b;
    return b;
}

struct Plan {
    int32_t tile_tokens, ntiles;
    size_t ws_e, ws_g;  // bytes of the two histogram arrays
};

// Tiles hold whole tokens (so a token's group-leader test stays inside one tile), at least
// ~512 slots each and at most 256 tiles, which keeps the single-workgroup scan short.
Plan make_plan(int64_t T, int32_t K, int32_t E, int32_t G)
{
    Plan p{};
    int64_t tt = ceil_div(512, K);
    tt = std::max<int64_t>(tt, ceil_div(T, 256));
    p.tile_tokens = static_cast<int32_t>(std::min<int64_t>(tt, 0x7fffffff));
    p.ntiles = static_cast<int32_t>(T == 0 ? 0 : ceil_div(T, p.tile_tokens));
    auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    p.ws_e = al(sizeof(int32_t) * static_cast<size_t>(E) * p.ntiles);
    p.ws_g = G > 0 ? al(sizeof(int32_t) * static_cast<size_t>(G) * p.ntiles) : 0;
    return p;
}

moe_status check_sizes(int64_t T, int32_t K, int32_t E, int32_t group_size)
{
    if (T < 0 || K < 1 || E < 1 || K > E)
        return MOE_ERR_INVALID;
    if (group_size > 0 && E % group_size != 0)
        return MOE_ERR_INVALID;
    if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (T * K > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_build_index_workspace_size(int64_t T, int32_t K, int32_t E,
                                                     int32_t group_size, size_t *bytes)
{
    using namespace moe;
    if (!bytes)
        return MOE_ERR_INVALID;
    const moe_status st = check_sizes(T, K, E, group_size);
    if (st != MOE_OK)
        return st;
    const Plan p = make_plan(T, K, E, group_size > 0 ? E / group_size : 0);
    *bytes = p.ws_e + p.ws_g;
    return MOE_OK;
}

extern "C" moe_status moe_build_index(const int32_t *topk_idx, const float *topk_w, int64_t T,
                                      int32_t K, int32_t E, int32_t capacity, int32_t group_size,
                                      const moe_index *out, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream)
{
    using namespace moe;
    moe_status st = check_sizes(T, K, E, group_size);
    if (st != MOE_OK)
        return st;
    if (capacity > 0 && group_size > 0)
        return MOE_ERR_UNSUPPORTED;
    if (capacity > 0 && static_cast<int64_t>(E) * capacity > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    // only the arrays that will be written must be present (empty tensors may come as NULL)
    const int32_t G = group_size > 0 ? E / group_size : 0;
    const int64_t R = capacity > 0 ? static_cast<int64_t>(E) * capacity : T * K;
    if (!out || !out->counts || !out->group_list || (R > 0 && !out->sorted_indices) ||
        (T > 0 && !out->row_of))
        return MOE_ERR_INVALID;
    if (G > 0 && (!out->group_counts || !out->n_slots ||
                  (T > 0 && (!out->slot_of || !out->gsrc || !out->esrc))))
        return MOE_ERR_INVALID;
    if (T > 0 && !topk_idx)
        return MOE_ERR_INVALID;
    const Plan p = make_plan(T, K, E, G);
    if (p.ntiles > 0 && (!workspace || workspace_bytes < p.ws_e + p.ws_g))
        return MOE_ERR_INVALID;

    IndexArgs a{};
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.T = T;
    a.K = K;
    a.E = E;
    a.cap = capacity > 0 ? capacity : 0;
    a.gs = group_size > 0 ? group_size : 0;
    a.G = G;
    a.tile_tokens = p.tile_tokens;
    a.ntiles = p.ntiles;
    a.ebits = bits_for(E);
    a.gbits = bits_for(G);
    a.hist_e = static_cast<int32_t *>(workspace);
    a.hist_g = G > 0 ? reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + p.ws_e) : nullptr;
    a.ix = *out;

    if (T == 0) {
        // nothing routed: the scan alone writes zero counts and the padding rows
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
        return launch_status();
    }

    const size_t lds_keys = sizeof(int32_t) * (static_cast<size_t>(E) + G);
    hipLaunchKernelGGL(hist_kernel, dim3(p.ntiles), dim3(256), lds_keys, stream, a);
    if ((st = launch_status()) != MOE_OK)
        return st;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
    if ((st = launch_status()) != MOE_OK)
        return st;
    hipLaunchKernelGGL(rank_kernel, dim3(p.ntiles), dim3(kWave), lds_keys, stream, a);
    if ((st = launch_status()) != MOE_OK)
        return st;
    if (G > 0) {
        const int64_t n = T * K;
        const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(n, 256), 4096));
        hipLaunchKernelGGL(esrc_kernel, dim3(blocks), dim3(256), 0, stream, a);
        if ((st = launch_status()) != MOE_OK)
            return st;
    }
    return MOE_OK;
}
