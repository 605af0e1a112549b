// Expert-major index build: a stable counting sort of the T*K routing slots by expert.
//
// Definition followed ([Megatron] §1.1, "token dispatcher + fuse_a2a", permute()): the routing
// map is transposed to [experts, tokens] and masked_select lists, expert by expert, the tokens
// routed there in ascending order -> sorted_indices; the same mask over the transposed probs
// gives permuted_probs; [Scratch] §7 ("从零理解 MoE 算子") gives group_list as the running sum
// of the per-expert counts. Ordering the slots i = t*K + k by (expert, i) is exactly that list.
//
// gfx950 design. A dependent global-memory round trip costs microseconds here, so every pass
// issues its loads together, stores whole cache lines, and orders loads before stores (on gfx9
// the vector-memory counter retires loads and stores in issue order, so a load issued after a
// store cannot be waited for without waiting for the store too). Two launches, plus one in
// group mode when K is not a power of two:
//   1. hist   one workgroup per tile of whole tokens: the tile's expert histogram (and the
//             group histogram of each token's first slot in a group) with LDS atomics -- only
//             counts come from atomics, never positions, so the result is deterministic -- and
//             one coalesced row per tile: the expert counts, then (group mode) the group
//             counts, so that the rank kernel gets both with one pass of loads.
//   2. rank   one workgroup per tile. It first adds up the tile counts of all tiles itself
//             (threads own 4 consecutive keys and a range of tiles, 16 loads in flight each;
//             the partial sums meet in LDS): every key's total, a block scan of the totals for
//             every key's first row, and the counts of the tiles before its own; tile 0 also
//             writes counts, group_list and the capacity bookkeeping. (A separate one-workgroup
//             scan launch between the two took 5.9 us at T16384 K8 E256, the rank kernel
//             re-reading its results.) Its tokens are split over 8 wavefronts (per-wave counts
//             and a prefix over the waves in LDS); each wavefront walks its slots 64 at a time
//             in slot order, in batches of 2 or 8 such groups (the smaller batch whenever it
//             holds a wave's slots: smaller code, see kRankBatchSmall). Lanes with the same key
//             find each other with one ballot per key bit (a match-any built from ballots); their
//             stable rank is popcount(peers & lanes_below) and the last peer advances the key's
//             running row counter in LDS. The workgroups then write the padding or unused rows
//             together.
//   3. esrc   (group mode, K not a power of two) expert-major row -> group slot (and routing
//             slot -> group slot, slot_src). With K a power
//             of two a token's slots sit in consecutive lanes of one wavefront: the first slot
//             of each (token, group) is found with ballots, and the rank kernel hands its group
//             slot to the token's other slots of the group and writes esrc itself.
// With no tokens one single-workgroup launch writes the zero counts and the marks; with at most
// one 512-slot batch per rank wavefront (T*K <= 4096) the rank kernel runs alone as one
// workgroup and takes the totals from its own per-wave counts; up to T*K = 16384 every rank
// workgroup counts all slots itself. Neither needs the histogram launch.
// The drop-and-pad capacity rule ([Scratch] §18, §26.6), the expert alignment ([Combine] §6:
// segments rounded up to a multiple of A with padding rows, the segment starts being the scan of
// the aligned lengths) and the group (send once per rank) slots ([CANN] §1(1)) are applied
// inside the same passes. Rows after the last segment are unused slack (MOE_ROW_UNUSED).
#include <algorithm>
#include <mutex>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxTiles = 128;      // tiles grow with T so that there are never more
constexpr int kEmptyThreads = 1024;
// 64-slot groups whose loads a rank wave issues together (a template argument of the rank
// kernel, 2 or 8): the rank kernel's batch loops are unrolled, and with caches flushed its code
// comes from HBM as it runs -- the group-mode kernel was 67 KB with 8 groups per batch and 27 KB
// with 2 (T8192 K8 E256 in 32 groups: 15.2 -> 12.0 us per launch; T16384 K8 E256: 8.6 -> 7.9 us).
// Waves with more slots take the larger batch (fewer dependent round trips: at T1048576 K8 the
// launch took 131 us with 8 groups per batch and 147 us with 2).
constexpr int kRankBatchSmall = 2;
constexpr int kRankBatchLarge = 8;

struct IndexArgs {
    const int32_t *topk_idx;
    const float *topk_w;
    int64_t T;
    int32_t K, E, cap, gs, G;
    int32_t align;   // expert alignment (1: none)
    int32_t Ep, Gp;  // E, G rounded up to a multiple of 4
    int32_t Hp;      // Ep + Gp (Gp only in group mode): the stride of a tile's row of counts
    int32_t tile_tokens, ntiles;
    int32_t ebits, gbits;
    int32_t *hist;    // [ntiles][Hp] tile counts: experts at [0, Ep), group slots at [Ep, Ep + Gp)
    moe_index ix;
};

__device__ __forceinline__ bool valid_expert(int e, int E) { return e >= 0 && e < E; }

__host__ __device__ __forceinline__ int64_t round_up(int64_t n, int64_t a) { return (n + a - 1) / a * a; }

// Rows of the expert-major buffer: E*cap with a capacity, otherwise T*K plus the most the
// aligned segments can add.
__host__ __device__ __forceinline__ int64_t index_rows(int64_t T, int32_t K, int32_t E, int32_t cap, int32_t align)
{
    return cap > 0 ? static_cast<int64_t>(E) * cap : T * K + static_cast<int64_t>(E) * (align - 1);
}

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

// group_leader by ballots, for a wavefront whose 64 lanes hold consecutive slots starting at a
// token boundary with K a power of two (so a token's K slots are lanes first .. first+K-1).
// `peers` are the valid lanes naming this lane's group (match_peers over the group ids);
// token_first gives the lowest of them inside this lane's token (64 if there is none), the lane
// holding the token's first slot in that group.
__device__ __forceinline__ int token_first(uint64_t peers, int K)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int first = lane & ~(K - 1);
    const uint64_t tok = K >= kWave ? ~0ull : ((1ull << K) - 1) << first;
    const uint64_t mine = peers & tok;
    return mine ? __builtin_ctzll(mine) : kWave;
}

// True iff the lane is valid and holds its token's first slot in its group.
__device__ __forceinline__ bool token_leader(uint64_t peers, bool valid, int K)
{
    return valid && token_first(peers, K) == static_cast<int>(threadIdx.x & (kWave - 1));
}

// ---------------------------------------------------------------- 1. per-tile histograms
constexpr int kHistThreads = 256;
constexpr int kHistLoads = 8;  // expert ids a thread has in flight (2 in group mode, see below)

// kGroups: group mode (a.gs > 0), a template argument so that the expert-only build carries no
// group code. A thread's ids are loaded several at a time, the next batch in flight while the
// current one is counted: one load and its wait per id took 113 us per launch at T1048576 K8
// (tiles of 256 ids per thread), 8 in flight 27 us; in group mode 2 in flight (T524288 K8, 32
// groups: 122 -> 81 us), because the unrolled group test of 8 made the kernel 14 KB instead of
// 2 KB and, with caches flushed, its code fetch cost 2.4 us per launch at T8192. No difference
// at T16384 K8 either way.
template <bool kGroups>
__global__ __launch_bounds__(kHistThreads) void hist_kernel(IndexArgs a)
{
    extern __shared__ int32_t sh[];
    int32_t *he = sh;         // [Ep]
    int32_t *hg = sh + a.Ep;  // [Gp]
    const int tile = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(tile) * a.tile_tokens;
    const int64_t t1 = min(a.T, t0 + a.tile_tokens);
    const int64_t s0 = t0 * a.K, s1 = t1 * a.K;
    constexpr int kLoads = kGroups ? 2 : kHistLoads;
    constexpr int64_t kStep = static_cast<int64_t>(kLoads) * kHistThreads;
    int nx[kLoads];
    auto load = [&](int64_t base) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int64_t i = base + u * kHistThreads + tid;
            nx[u] = i < s1 ? a.topk_idx[i] : -1;
        }
    };
    load(s0);
    const int nsh = a.Ep + (kGroups ? a.Gp : 0);
    for (int i = tid; i < nsh; i += kHistThreads)
        sh[i] = 0;
    __syncthreads();
    // with K a power of two each wavefront's 64 slots start at a token boundary (s0, 64 and the
    // workgroup's stride are multiples of K) and the group test runs on ballots; every lane takes
    // part in the ballots, the ones past s1 as invalid slots of whole tokens
    const bool wave_lead = (a.K & (a.K - 1)) == 0;
    for (int64_t base = s0; base < s1; base += kStep) {
        int ids[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            ids[u] = nx[u];
        if (base + kStep < s1)
            load(base + kStep);
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int64_t i = base + u * kHistThreads + tid;
            const int e = ids[u];
            const bool ok = i < s1 && valid_expert(e, a.E);
            bool lead = false;
            if (kGroups && wave_lead)
                lead = token_leader(match_peers(ok ? e / a.gs : -1, a.gbits, __ballot(ok)), ok, a.K);
            if (!ok)
                continue;
            atomicAdd(&he[e], 1);
            if (kGroups) {
                const int64_t t = i / a.K;
                const int k = static_cast<int>(i - t * a.K);
                const int g = e / a.gs;
                if (wave_lead ? lead : group_leader(a.topk_idx + t * a.K, k, g, a.E, a.gs))
                    atomicAdd(&hg[g], 1);
            }
        }
    }
    if (kGroups) {  // slot_of starts as "absent" for this tile's tokens
        for (int64_t i = t0 * a.G + tid; i < t1 * a.G; i += kHistThreads)
            a.ix.slot_of[i] = -1;
    }
    __syncthreads();
    int32_t *row = a.hist + static_cast<int64_t>(tile) * a.Hp;  // expert and group counts, one row
    for (int i = tid; i < a.Hp; i += kHistThreads)
        row[i] = sh[i];
}

// ---------------------------------------------------------------- no tokens
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t u = __shfl_up(v, off, kWave);
        if (lane >= off)
            v += u;
    }
    return v;
}

// T == 0: zero counts and group_list (every segment is empty), and every row marked -- padding
// in drop-and-pad, unused slack otherwise.
__global__ __launch_bounds__(kEmptyThreads) void empty_index_kernel(IndexArgs a)
{
    const int tid = threadIdx.x;
    for (int e = tid; e < a.E; e += kEmptyThreads) {
        a.ix.counts[e] = 0;
        a.ix.group_list[e] = 0;
        if (a.ix.kept_counts)
            a.ix.kept_counts[e] = 0;
    }
    const int64_t R = index_rows(a.T, a.K, a.E, a.cap, a.align);
    const int32_t mark = a.cap > 0 ? MOE_ROW_PAD : MOE_ROW_UNUSED;
    for (int64_t r = tid; r < R; r += kEmptyThreads) {
        a.ix.sorted_indices[r] = mark;
        if (a.ix.permuted_probs)
            a.ix.permuted_probs[r] = 0.0f;
        if (a.gs > 0)
            a.ix.esrc[r] = mark;
    }
    if (a.gs > 0) {
        for (int g = tid; g < a.G; g += kEmptyThreads)
            a.ix.group_counts[g] = 0;
        if (tid == 0)
            a.ix.n_slots[0] = 0;
    }
}

// ---------------------------------------------------------------- 2. stable ranks

__device__ __forceinline__ int last_lane(uint64_t m) { return 63 - __clzll(m); }

// a tile's tokens are split across 8 wavefronts (at T16384 K8 E256: 10.2 us per launch, 13.3 us
// with 4; more and smaller tiles did not help)
constexpr int kRankWaves = 8;
constexpr int kRankThreads = kRankWaves * kWave;
constexpr int kSpanLarge = kRankBatchLarge * kWave;  // slots whose loads a wavefront issues together
// up to this many routed slots (one batch per wavefront) the index is built by one workgroup
// in one launch: T1024 K2 E8 0.030 -> 0.025 ms per step; at T4096 K2 E64 (two batches per
// wavefront) the single workgroup lost, 0.061 against 0.055 ms
constexpr int64_t kSingleTileSlots = static_cast<int64_t>(kRankWaves) * kSpanLarge;

// True when slot i = (t, k) is the first of token t's slots in group g. The token's earlier
// slots are in `ids` (the current batch, starting at slot base0) or, when the token straddles
// the batch start, just before it.
__device__ __forceinline__ bool first_in_group(const IndexArgs &a, int64_t i, int k, int g, int64_t base0,
                                               const int32_t *ids)
{
    bool lead = true;
    for (int j = 1; j <= k; ++j) {
        const int64_t q = i - j;
        const int ej = q >= base0 ? ids[q - base0] : a.topk_idx[q];
        if (valid_expert(ej, a.E) && ej / a.gs == g)
            lead = false;
    }
    return lead;
}

template <int RB>
__device__ __forceinline__ void load_batch(const IndexArgs &a, int64_t base0, int64_t s1, bool want_w, int (&e)[RB],
                                           float (&w)[RB])
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const int64_t i = base0 + b * kWave + lane;
        e[b] = i < s1 ? a.topk_idx[i] : -1;
        w[b] = want_w && i < s1 ? a.topk_w[i] : 1.0f;
    }
}

constexpr int kOffsetLoads = 16;  // tile-count vectors a thread has in flight
// ints of the per-wave id buffers, which tile_sums also uses for its partial sums
constexpr int ids_ints(int rb)
{
    return kRankWaves * rb * kWave > 2 * 4 * kRankThreads ? kRankWaves * rb * kWave : 2 * 4 * kRankThreads;
}

// Per key of the tile counts hist[0..ntiles)[0..nkeys) (rows of `stride` keys, 16-byte aligned):
// tot[key] = the sum over all tiles, pre[key] = the sum over the tiles before `tile`. A thread
// owns 4 consecutive keys and a contiguous range of tiles; the ranges' partial sums meet in LDS
// (`scratch`: 2 * kRankThreads * 4 ints) and are added in range order. Ends with a barrier.
__device__ void tile_sums(const int32_t *hist, int nkeys, int stride, int ntiles, int tile, int32_t *tot,
                          int32_t *pre, int32_t *scratch)
{
    const int tid = threadIdx.x;
    const int nq = stride / 4;             // stride is a multiple of 4 and at most 4 * kRankThreads
    const int splits = kRankThreads / nq;  // tile ranges
    const int q = tid % nq, r = tid / nq;
    const int tps = (ntiles + splits - 1) / splits;
    int32_t *part_tot = scratch;                   // [splits][stride]
    int32_t *part_pre = scratch + splits * stride;  // [splits][stride]
    if (r < splits) {
        const int j0 = r * tps, j1 = min(ntiles, j0 + tps);
        u32x4 st{0u, 0u, 0u, 0u}, sp{0u, 0u, 0u, 0u};
        for (int jb = j0; jb < j1; jb += kOffsetLoads) {
            u32x4 c[kOffsetLoads];
#pragma unroll
            for (int u = 0; u < kOffsetLoads; ++u)
                c[u] = jb + u < j1 ? ld16(hist + static_cast<int64_t>(jb + u) * stride + 4 * q) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < kOffsetLoads; ++u) {
                const bool before = jb + u < tile;
                st.x += c[u].x;
                st.y += c[u].y;
                st.z += c[u].z;
                st.w += c[u].w;
                sp.x += before ? c[u].x : 0u;
                sp.y += before ? c[u].y : 0u;
                sp.z += before ? c[u].z : 0u;
                sp.w += before ? c[u].w : 0u;
            }
        }
        int32_t *pt = part_tot + r * stride + 4 * q;
        int32_t *pp = part_pre + r * stride + 4 * q;
        pt[0] = static_cast<int32_t>(st.x);
        pt[1] = static_cast<int32_t>(st.y);
        pt[2] = static_cast<int32_t>(st.z);
        pt[3] = static_cast<int32_t>(st.w);
        pp[0] = static_cast<int32_t>(sp.x);
        pp[1] = static_cast<int32_t>(sp.y);
        pp[2] = static_cast<int32_t>(sp.z);
        pp[3] = static_cast<int32_t>(sp.w);
    }
    __syncthreads();
    for (int key = tid; key < nkeys; key += kRankThreads) {
        int32_t t = 0, p = 0;
        for (int rr = 0; rr < splits; ++rr) {
            t += part_tot[rr * stride + key];
            p += part_pre[rr * stride + key];
        }
        tot[key] = t;
        pre[key] = p;
    }
    __syncthreads();
}

// seg[key] = the sum of round_up(tot, align) over the keys before it (nkeys <= 4 * kRankThreads;
// each thread takes 4 consecutive keys); returns the sum over all keys. Ends with a barrier.
__device__ int32_t segment_starts(const int32_t *tot, int nkeys, int align, int32_t *seg, int32_t *wsum)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int k0 = 4 * tid;
    int32_t v[4];
    int32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = k0 + i < nkeys ? static_cast<int32_t>(round_up(tot[k0 + i], align)) : 0;
        sum += v[i];
    }
    const int32_t inc = wave_inclusive_scan(sum);
    if (lane == kWave - 1)
        wsum[wave] = inc;
    __syncthreads();
    int32_t run = inc - sum, total = 0;
    for (int w = 0; w < kRankWaves; ++w) {
        run += w < wave ? wsum[w] : 0;
        total += wsum[w];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (k0 + i < nkeys)
            seg[k0 + i] = run;
        run += v[i];
    }
    __syncthreads();
    return total;
}

// Up to this many routed slots every rank workgroup counts all of them itself (kCountAll) instead
// of reading the tile counts of a histogram launch: each small launch costs ~4 us with cold caches
// (T4096 K2 E64: histogram 4.4 us + ranks 8.2 us), far more than 16 loads and LDS atomics per
// thread.
constexpr int64_t kCountAllSlots = 16384;
constexpr int kCountLoads = 16;  // ids a thread has in flight while counting all slots

// kCountAll: per key, tot = the slots of all tokens (experts) or their first slots in each group
// (groups, at Ep), pre = those of the tokens before this tile (slots below tile_s0). tot and pre
// are adjacent in LDS (pre = tot + Hp). Counts come from LDS atomics, positions never do. Ends with
// a barrier.
template <bool kGroups>
__device__ void count_all(const IndexArgs &a, int64_t tile_s0, int32_t *tot)
{
    int32_t *pre = tot + a.Hp;
    const int tid = threadIdx.x;
    const int64_t n = a.T * a.K;
    constexpr int64_t kStep = static_cast<int64_t>(kCountLoads) * kRankThreads;
    int nx[kCountLoads];  // the next batch, in flight while the current one is counted
    auto load = [&](int64_t base) {
#pragma unroll
        for (int u = 0; u < kCountLoads; ++u) {
            const int64_t i = base + u * kRankThreads + tid;
            nx[u] = i < n ? a.topk_idx[i] : -1;
        }
    };
    load(0);
    for (int i = tid; i < 2 * a.Hp; i += kRankThreads)
        tot[i] = 0;
    __syncthreads();
    // with K a power of two each wavefront's 64 slots start at a token boundary, so the group
    // test runs on ballots; every lane takes part, the ones past n as invalid slots
    const bool wave_lead = (a.K & (a.K - 1)) == 0;
    for (int64_t base = 0; base < n; base += kStep) {
        int ids[kCountLoads];
#pragma unroll
        for (int u = 0; u < kCountLoads; ++u)
            ids[u] = nx[u];
        if (base + kStep < n)
            load(base + kStep);
#pragma unroll
        for (int u = 0; u < kCountLoads; ++u) {
            const int64_t i = base + u * kRankThreads + tid;
            const int e = ids[u];
            const bool ok = i < n && valid_expert(e, a.E);
            bool lead = false;
            if (kGroups && wave_lead)
                lead = token_leader(match_peers(ok ? e / a.gs : -1, a.gbits, __ballot(ok)), ok, a.K);
            if (!ok)
                continue;
            const bool before = i < tile_s0;
            atomicAdd(&tot[e], 1);
            if (before)
                atomicAdd(&pre[e], 1);
            if (kGroups) {
                const int64_t t = i / a.K;
                const int k = static_cast<int>(i - t * a.K);
                const int g = e / a.gs;
                if (wave_lead ? lead : group_leader(a.topk_idx + t * a.K, k, g, a.E, a.gs)) {
                    atomicAdd(&tot[a.Ep + g], 1);
                    if (before)
                        atomicAdd(&pre[a.Ep + g], 1);
                }
            }
        }
    }
    __syncthreads();
}

// One workgroup per tile, kRankWaves wavefronts, each owning a contiguous share of the tile's
// tokens (whole tokens). Phase A: every wave counts its slots per expert (and its first-in-group
// slots per group) in LDS. Phase B: per key, a prefix over the waves starting at the tile's
// first row of the key. Phase C: every wave walks its slots in order, 64 at a time, and ranks
// them against its own running counters. Finally the workgroups together write the padding
// (drop-and-pad) or unused rows.
// kTotals says where the per-key totals come from: kFromTiles, the tile counts of the histogram
// launch; kSingle, one workgroup holding all tokens (small inputs), its own per-wave counts after
// phase A; kCountAll, every workgroup counting all slots itself (small inputs, no histogram launch).
constexpr int kFromTiles = 0, kSingle = 1, kCountAll = 2;
template <bool kGroups, int kTotals, int RB>
__global__ __launch_bounds__(kRankThreads) void rank_kernel(IndexArgs a)
{
    constexpr int kSpan = RB * kWave;  // slots of one batch of a wave
    extern __shared__ int32_t sh[];
    __shared__ int32_t wsum[kRankWaves];
    int32_t *cnt_e = sh;                        // [kRankWaves][E] counts -> next row of the wave
    int32_t *cnt_g = cnt_e + kRankWaves * a.E;  // [kRankWaves][G]
    int32_t *seg_e = cnt_g + kRankWaves * a.G;  // [E] first row of each expert
    int32_t *seg_g = seg_e + a.E;               // [G] first slot of each group
    int32_t *tot = seg_g + a.G;                 // [Hp] slots per key: experts, then groups at Ep
    int32_t *pre = tot + a.Hp;                  // [Hp] of those, the ones in tiles before this one
    int32_t *tot_e = tot, *pre_e = pre;
    int32_t *tot_g = tot + a.Ep, *pre_g = pre + a.Ep;
    int32_t *ids_all = pre + a.Hp;  // [kRankWaves][kSpan] expert ids of each wave's batch (first: sums)
    const int tile = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    int32_t *cw_e = cnt_e + wave * a.E;
    int32_t *cw_g = cnt_g + wave * a.G;
    int32_t *ids = ids_all + wave * kSpan;
    for (int i = tid; i < kRankWaves * (a.E + a.G); i += kRankThreads)
        sh[i] = 0;

    // this wave's tokens and slots
    const int64_t tile_t0 = static_cast<int64_t>(tile) * a.tile_tokens;
    const int64_t tile_t1 = min(a.T, tile_t0 + a.tile_tokens);
    const int64_t per = (a.tile_tokens + kRankWaves - 1) / kRankWaves;
    const int64_t t0 = min(tile_t1, tile_t0 + wave * per);
    const int64_t t1 = min(tile_t1, t0 + per);
    const int64_t s0 = t0 * a.K, s1 = t1 * a.K;
    // K a power of two: every batch of 64 slots starts at a token boundary (s0 and kWave are
    // multiples of K), so the first-slot-in-group test runs on ballots instead of reading the
    // token's earlier slots back from LDS
    const bool wave_lead = (a.K & (a.K - 1)) == 0;
    const bool want_w = a.ix.permuted_probs && a.topk_w;
    int e_first[RB];
    float w_first[RB];
    load_batch(a, s0, s1, want_w, e_first, w_first);

    // every key's first row from the totals; tile 0 writes the per-expert (and per-group) results
    int32_t rows_used = 0;
    auto segments = [&]() {
        rows_used = segment_starts(tot_e, a.E, a.cap > 0 ? 1 : a.align, seg_e, wsum);
        int32_t n_slots = 0;
        if (kGroups)
            n_slots = segment_starts(tot_g, a.G, 1, seg_g, wsum);
        if (tile == 0) {
            for (int e = tid; e < a.E; e += kRankThreads) {
                const int32_t cnt = tot_e[e];
                a.ix.counts[e] = cnt;
                a.ix.group_list[e] = seg_e[e] + (a.cap > 0 ? cnt : static_cast<int32_t>(round_up(cnt, a.align)));
                if (a.ix.kept_counts)
                    a.ix.kept_counts[e] = a.cap > 0 ? min(cnt, a.cap) : cnt;
            }
            if (kGroups) {
                for (int g = tid; g < a.G; g += kRankThreads)
                    a.ix.group_counts[g] = tot_g[g];
                if (tid == 0)
                    a.ix.n_slots[0] = n_slots;
            }
        }
    };
    if constexpr (kTotals == kSingle) {
        if (kGroups) {  // slot_of starts as "absent" (the histogram kernel does this otherwise)
            for (int64_t i = tid; i < a.T * a.G; i += kRankThreads)
                a.ix.slot_of[i] = -1;
        }
        __syncthreads();  // the zeroed counters before phase A's atomics
    } else if constexpr (kTotals == kCountAll) {
        if (kGroups) {  // slot_of starts as "absent" for this tile's tokens
            for (int64_t i = tile_t0 * a.G + tid; i < tile_t1 * a.G; i += kRankThreads)
                a.ix.slot_of[i] = -1;
        }
        count_all<kGroups>(a, tile_t0 * a.K, tot);  // its barriers also cover the zeroed counters
        segments();
    } else {
        // the totals, and this tile's first row inside each key, from the tile counts (each
        // workgroup adds up the counts of all tiles itself: no separate scan pass; expert and
        // group counts share a row, so one pass of loads covers both)
        tile_sums(a.hist, a.Hp, a.Hp, a.ntiles, tile, tot, pre, ids_all);
        segments();
    }

    // ---- phase A: per-wave counts
    for (int64_t base0 = s0; base0 < s1; base0 += kSpan) {
        int e_b[RB];
        float w_b[RB];
        if (base0 == s0) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
                e_b[b] = e_first[b];
        } else {
            load_batch(a, base0, s1, false, e_b, w_b);
        }
        if (kGroups && !wave_lead) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
                ids[b * kWave + lane] = e_b[b];
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int64_t i = base0 + b * kWave + lane;
            const int e = e_b[b];
            const bool ok = i < s1 && valid_expert(e, a.E);
            bool lead = false;
            if (kGroups && wave_lead)
                lead = token_leader(match_peers(ok ? e / a.gs : -1, a.gbits, __ballot(ok)), ok, a.K);
            if (!ok)
                continue;
            atomicAdd(&cw_e[e], 1);
            if (kGroups) {
                const int64_t t = i / a.K;
                const int k = static_cast<int>(i - t * a.K);
                const int g = e / a.gs;
                if (wave_lead ? lead : first_in_group(a, i, k, g, base0, ids))
                    atomicAdd(&cw_g[g], 1);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    if constexpr (kTotals == kSingle) {  // the totals are this workgroup's own counts
        for (int e = tid; e < a.E; e += kRankThreads) {
            int32_t sum = 0;
            for (int w = 0; w < kRankWaves; ++w)
                sum += cnt_e[w * a.E + e];
            tot_e[e] = sum;
            pre_e[e] = 0;
        }
        if (kGroups) {
            for (int g = tid; g < a.G; g += kRankThreads) {
                int32_t sum = 0;
                for (int w = 0; w < kRankWaves; ++w)
                    sum += cnt_g[w * a.G + g];
                tot_g[g] = sum;
                pre_g[g] = 0;
            }
        }
        __syncthreads();
        segments();
    }

    // ---- phase B: each wave's first row per key
    {
        for (int e = tid; e < a.E; e += kRankThreads) {
            int32_t run = seg_e[e] + pre_e[e];
            for (int w = 0; w < kRankWaves; ++w) {
                const int32_t c = cnt_e[w * a.E + e];
                cnt_e[w * a.E + e] = run;
                run += c;
            }
        }
        if (kGroups) {
            for (int g = tid; g < a.G; g += kRankThreads) {
                int32_t run = seg_g[g] + pre_g[g];
                for (int w = 0; w < kRankWaves; ++w) {
                    const int32_t c = cnt_g[w * a.G + g];
                    cnt_g[w * a.G + g] = run;
                    run += c;
                }
            }
        }
    }
    __syncthreads();

    // ---- phase C: stable ranks
    const uint64_t below = lanemask_lt();
    int e_nx[RB];
    float w_nx[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        e_nx[b] = e_first[b];
        w_nx[b] = w_first[b];
    }
    for (int64_t base0 = s0; base0 < s1; base0 += kSpan) {
        int e_cur[RB];
        float w_cur[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            e_cur[b] = e_nx[b];
            w_cur[b] = w_nx[b];
        }
        if (base0 + kSpan < s1)  // next batch in flight, issued before this batch's stores
            load_batch(a, base0 + kSpan, s1, want_w, e_nx, w_nx);
        if (kGroups && !wave_lead) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
                ids[b * kWave + lane] = e_cur[b];
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            if (base0 + b * kWave >= s1)
                break;
            const int64_t i = base0 + b * kWave + lane;
            const bool in = i < s1;
            const int e = e_cur[b];
            const bool ok = in && valid_expert(e, a.E);
            const int64_t t = i / a.K;
            const int k = static_cast<int>(i - t * a.K);

            // expert-major row
            const uint64_t pe = match_peers(e, a.ebits, __ballot(ok));
            int32_t row = -1;
            if (ok) {
                const int32_t r = cw_e[e] + __popcll(pe & below);
                row = r;
                if (a.cap > 0) {
                    const int32_t p = r - seg_e[e];  // position inside the expert
                    row = p < a.cap ? e * a.cap + p : -1;
                }
            }
            __builtin_amdgcn_wave_barrier();
            if (ok && lane == last_lane(pe))
                cw_e[e] += __popcll(pe);
            if (in)
                a.ix.row_of[i] = row;
            if (row >= 0) {
                a.ix.sorted_indices[row] = static_cast<int32_t>(t);
                if (a.ix.permuted_probs)
                    a.ix.permuted_probs[row] = w_cur[b];
            }

            // group slots: one per (token, group), listed group by group, tokens ascending
            if (kGroups) {
                const int g = ok ? e / a.gs : -1;
                bool lead;
                uint64_t pg;
                int from = lane;  // the lane that gets this slot's group slot (wave_lead)
                if (wave_lead) {
                    const uint64_t peers = match_peers(g, a.gbits, __ballot(ok));
                    if (ok)
                        from = token_first(peers, a.K);
                    lead = ok && from == lane;
                    pg = peers & __ballot(lead);
                } else {
                    lead = ok && first_in_group(a, i, k, g, base0, ids);
                    pg = match_peers(g, a.gbits, __ballot(lead));
                }
                int32_t slot = -1;
                if (lead)
                    slot = cw_g[g] + __popcll(pg & below);
                __builtin_amdgcn_wave_barrier();
                if (lead && lane == last_lane(pg))
                    cw_g[g] += __popcll(pg);
                if (wave_lead) {  // every kept slot of the group takes the leader's group slot
                    const int32_t gslot = __shfl(slot, from, kWave);
                    if (row >= 0)
                        a.ix.esrc[row] = gslot;
                    if (in && a.ix.slot_src)
                        a.ix.slot_src[i] = row >= 0 ? gslot : -1;
                }
                if (lead) {
                    a.ix.slot_of[t * a.G + g] = slot;
                    a.ix.gsrc[slot] = static_cast<int32_t>(t);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- padding rows (drop-and-pad) or rows after the last routed slot
    const int32_t *cnt = tot_e;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kRankThreads;
    if (a.cap > 0) {
        const int64_t R = static_cast<int64_t>(a.E) * a.cap;
        for (int64_t r = static_cast<int64_t>(tile) * kRankThreads + tid; r < R; r += stride) {
            const int e = static_cast<int>(r / a.cap);
            const int p = static_cast<int>(r - static_cast<int64_t>(e) * a.cap);
            if (p >= min(cnt[e], a.cap)) {
                a.ix.sorted_indices[r] = MOE_ROW_PAD;
                if (a.ix.permuted_probs)
                    a.ix.permuted_probs[r] = 0.0f;
            }
        }
    } else {
        const int A = a.align;
        if (A > 1) {  // padding rows at the end of each aligned segment: (expert, p) pairs
            const int64_t npad = static_cast<int64_t>(a.E) * (A - 1);
            for (int64_t j = static_cast<int64_t>(tile) * kRankThreads + tid; j < npad; j += stride) {
                const int e = static_cast<int>(j / (A - 1));
                const int p = static_cast<int>(j - static_cast<int64_t>(e) * (A - 1));
                const int32_t c = cnt[e];
                if (p < round_up(c, A) - c) {
                    const int64_t r = static_cast<int64_t>(seg_e[e]) + c + p;
                    a.ix.sorted_indices[r] = MOE_ROW_PAD;
                    if (a.ix.permuted_probs)
                        a.ix.permuted_probs[r] = 0.0f;
                    if (kGroups)
                        a.ix.esrc[r] = MOE_ROW_PAD;
                }
            }
        }
        const int64_t total = rows_used;
        const int64_t R = index_rows(a.T, a.K, a.E, 0, A);
        for (int64_t r = total + static_cast<int64_t>(tile) * kRankThreads + tid; r < R; r += stride) {
            a.ix.sorted_indices[r] = MOE_ROW_UNUSED;
            if (a.ix.permuted_probs)
                a.ix.permuted_probs[r] = 0.0f;
            if (kGroups)
                a.ix.esrc[r] = MOE_ROW_UNUSED;
        }
    }
}

// ---------------------------------------------------------------- 3. group mode: esrc
__global__ __launch_bounds__(256) void esrc_kernel(IndexArgs a)
{
    const int64_t n = a.T * a.K;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int e = a.topk_idx[i];
        const int32_t row = a.ix.row_of[i];
        const bool ok = valid_expert(e, a.E) && row >= 0;
        const int64_t t = i / a.K;
        const int32_t slot = ok ? a.ix.slot_of[t * a.G + e / a.gs] : -1;
        if (ok)
            a.ix.esrc[row] = slot;
        if (a.ix.slot_src)
            a.ix.slot_src[i] = slot;
    }
}

int bits_for(int n)  // bits needed to tell apart the keys 0..n-1
{
    int b = 0;
    while ((1 << b) < n)
        ++b;
    return b;
}

int round4(int n) { return (n + 3) & ~3; }

// rank_kernel<groups, totals, batch> for runtime choices of the three
template <bool kGroups, int kTotals>
void launch_rank_rb(int rb, dim3 grid, size_t lds, hipStream_t stream, const IndexArgs &a)
{
    if (rb == kRankBatchSmall)
        hipLaunchKernelGGL((rank_kernel<kGroups, kTotals, kRankBatchSmall>), grid, dim3(kRankThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((rank_kernel<kGroups, kTotals, kRankBatchLarge>), grid, dim3(kRankThreads), lds, stream, a);
}

template <bool kGroups>
void launch_rank_totals(int totals, int rb, dim3 grid, size_t lds, hipStream_t stream, const IndexArgs &a)
{
    if (totals == kSingle)
        launch_rank_rb<kGroups, kSingle>(rb, grid, lds, stream, a);
    else if (totals == kCountAll)
        launch_rank_rb<kGroups, kCountAll>(rb, grid, lds, stream, a);
    else
        launch_rank_rb<kGroups, kFromTiles>(rb, grid, lds, stream, a);
}

void launch_rank(bool groups, int totals, int rb, dim3 grid, size_t lds, hipStream_t stream, const IndexArgs &a)
{
    if (groups)
        launch_rank_totals<true>(totals, rb, grid, lds, stream, a);
    else
        launch_rank_totals<false>(totals, rb, grid, lds, stream, a);
}

struct Plan {
    int32_t tile_tokens, ntiles;
    size_t ws;  // workspace bytes: the tile counts
};

// Tiles hold whole tokens (so a token's group test stays inside one tile), at least ~512 slots
// each and at most kMaxTiles of them.
Plan make_plan(int64_t T, int32_t K, int32_t E, int32_t G)
{
    Plan p{};
    int64_t tt = ceil_div(512, K);
    tt = std::max<int64_t>(tt, ceil_div(T, kMaxTiles));
    p.tile_tokens = static_cast<int32_t>(std::min<int64_t>(tt, 0x7fffffff));
    p.ntiles = static_cast<int32_t>(T == 0 ? 0 : ceil_div(T, p.tile_tokens));
    auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    p.ws = al(sizeof(int32_t) * static_cast<size_t>(round4(E) + (G > 0 ? round4(G) : 0)) * p.ntiles);
    return p;
}

// The plan of tile counts written by the fused route kernel: tiles of tile_tokens tokens.
constexpr int kMaxCountedTiles = 256;
Plan counted_plan(int64_t T, int32_t E, int32_t G, int32_t tile_tokens)
{
    Plan p{};
    p.tile_tokens = tile_tokens;
    p.ntiles = static_cast<int32_t>(T == 0 ? 0 : ceil_div(T, tile_tokens));
    auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
    p.ws = al(sizeof(int32_t) * static_cast<size_t>(round4(E) + (G > 0 ? round4(G) : 0)) * p.ntiles);
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
    *bytes = p.ws;
    return MOE_OK;
}

extern "C" int64_t moe_index_rows(int64_t T, int32_t K, int32_t E, int32_t capacity, int32_t alignment)
{
    using namespace moe;
    if (T < 0 || K < 1 || E < 1 || alignment < 0 || (capacity > 0 && alignment > 1))
        return -1;
    const int64_t R = index_rows(T, K, E, capacity > 0 ? capacity : 0, alignment > 1 ? alignment : 1);
    return R > 0x7fffffffLL ? -1 : R;
}

namespace moe {
namespace {

// Argument checks, then (launch = true) the launches; `workspace` holds at least the plan's tile
// counts. With launch = false only the arguments other than the workspace are checked.
moe_status build_index_impl(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K, int32_t E,
                            int32_t capacity, int32_t group_size, int32_t alignment, const moe_index *out,
                            void *workspace, size_t workspace_bytes, hipStream_t stream, bool launch = true,
                            int32_t counted_tile_tokens = 0)
{
    moe_status st = check_sizes(T, K, E, group_size);
    if (st != MOE_OK)
        return st;
    if (alignment < 0)
        return MOE_ERR_INVALID;
    if (capacity > 0 && (group_size > 0 || alignment > 1))
        return MOE_ERR_UNSUPPORTED;
    const int32_t A = alignment > 1 ? alignment : 1;
    // only the arrays that will be written must be present (empty tensors may come as NULL)
    const int32_t G = group_size > 0 ? E / group_size : 0;
    const int64_t R = index_rows(T, K, E, capacity > 0 ? capacity : 0, A);
    if (R > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    if (!out || !out->counts || !out->group_list || (R > 0 && !out->sorted_indices) ||
        (T > 0 && !out->row_of))
        return MOE_ERR_INVALID;
    if (G > 0 && (!out->group_counts || !out->n_slots || (T > 0 && (!out->slot_of || !out->gsrc)) ||
                  (R > 0 && !out->esrc)))
        return MOE_ERR_INVALID;
    if (T > 0 && !topk_idx)
        return MOE_ERR_INVALID;
    // counted_tile_tokens > 0: the tile counts are already in the workspace (tiles of that many
    // tokens, counted by the fused route kernel), and only the rank pass is launched
    const Plan p = counted_tile_tokens > 0 ? counted_plan(T, E, G, counted_tile_tokens) : make_plan(T, K, E, G);
    if (p.ntiles > (counted_tile_tokens > 0 ? kMaxCountedTiles : kMaxTiles))
        return MOE_ERR_UNSUPPORTED;  // cannot happen: tiles grow with T to stay within the limit
    const size_t need = p.ws;
    if (!launch)
        return MOE_OK;
    if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace))))
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
    a.align = A;
    a.Ep = round4(E);
    a.Gp = round4(G);
    a.Hp = a.Ep + (G > 0 ? a.Gp : 0);
    a.tile_tokens = p.tile_tokens;
    a.ntiles = p.ntiles;
    a.ebits = bits_for(E);
    a.gbits = bits_for(G);
    char *ws = static_cast<char *>(workspace);
    a.hist = reinterpret_cast<int32_t *>(ws);
    a.ix = *out;

    if (T == 0) {
        // nothing routed: zero counts and the padding or unused marks
        hipLaunchKernelGGL(empty_index_kernel, dim3(1), dim3(kEmptyThreads), 0, stream, a);
        return launch_status();
    }

    const bool single = counted_tile_tokens == 0 && T * K <= kSingleTileSlots;  // one workgroup, one launch
    if (single) {
        a.tile_tokens = static_cast<int32_t>(T);
        a.ntiles = 1;
    }
    // the smaller batch when one batch of it holds each rank wave's slots
    const int64_t wave_slots = ceil_div(a.tile_tokens, kRankWaves) * K;
    const int rb = wave_slots <= static_cast<int64_t>(kRankBatchSmall) * kWave ? kRankBatchSmall : kRankBatchLarge;
    const size_t lds_rank = sizeof(int32_t) * (static_cast<size_t>(kRankWaves + 1) * (E + G) + 2 * static_cast<size_t>(a.Hp) +
                                               static_cast<size_t>(ids_ints(rb)));
    const int totals = counted_tile_tokens > 0 ? kFromTiles
                       : (single ? kSingle : (T * K <= kCountAllSlots ? kCountAll : kFromTiles));
    if (totals == kFromTiles && counted_tile_tokens == 0) {
        const size_t lds_hist = sizeof(int32_t) * static_cast<size_t>(a.Hp);
        if (G > 0)
            hipLaunchKernelGGL(hist_kernel<true>, dim3(p.ntiles), dim3(kHistThreads), lds_hist, stream, a);
        else
            hipLaunchKernelGGL(hist_kernel<false>, dim3(p.ntiles), dim3(kHistThreads), lds_hist, stream, a);
        if ((st = launch_status()) != MOE_OK)
            return st;
    }
    launch_rank(G > 0, totals, rb, dim3(static_cast<unsigned>(a.ntiles)), lds_rank, stream, a);
    if ((st = launch_status()) != MOE_OK)
        return st;
    if (G > 0 && (K & (K - 1)) != 0) {  // with K a power of two the rank kernel writes esrc
        const int64_t n = T * K;
        const int blocks = static_cast<int>(std::min<int64_t>(ceil_div(n, 256), 4096));
        hipLaunchKernelGGL(esrc_kernel, dim3(blocks), dim3(256), 0, stream, a);
        if ((st = launch_status()) != MOE_OK)
            return st;
    }
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_build_index(const int32_t *topk_idx, const float *topk_w, int64_t T,
                                      int32_t K, int32_t E, int32_t capacity, int32_t group_size,
                                      int32_t alignment, const moe_index *out, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream)
{
    return moe::build_index_impl(topk_idx, topk_w, T, K, E, capacity, group_size, alignment, out, workspace,
                                 workspace_bytes, stream);
}

namespace moe {

moe_status build_index_from_tile_counts(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K, int32_t E,
                                        int32_t capacity, int32_t group_size, int32_t alignment, const moe_index *out,
                                        void *workspace, size_t workspace_bytes, int32_t tile_tokens, bool launch,
                                        hipStream_t stream)
{
    if (tile_tokens < 1)
        return MOE_ERR_INVALID;
    return build_index_impl(topk_idx, topk_w, T, K, E, capacity, group_size, alignment, out, workspace,
                            workspace_bytes, stream, launch, tile_tokens);
}

bool build_index_counts_tiles(int64_t T, int32_t K) { return T * K > kCountAllSlots; }

}  // namespace moe

// ---------------------------------------------------------------- allocation-free entry point
// The tile counts of moe_build_index_noalloc live in this array instead of a caller's workspace:
// room for the largest plan any valid input makes (kMaxTiles tiles of MOE_MAX_EXPERTS expert
// counts and MOE_MAX_EXPERTS group counts, 4 bytes each: 1 MiB). Each GPU the library runs on holds
// its own copy until the process ends. The counts are written before they are read in every
// call, so nothing needs clearing between calls.
constexpr size_t kScratchBytes = sizeof(int32_t) * moe::kMaxTiles * (2 * MOE_MAX_EXPERTS);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxScratchDevices];  // device address of `scratch` per device, resolved once

// Device address of this device's copy of `scratch` (the array's name is only a host-side stand-in
// for it). Resolved on the first call on each device, with that device current.
moe_status scratch_address(int device, void **p)
{
    if (device < 0 || device >= kMaxScratchDevices)
        return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[device]) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
            return MOE_ERR_HIP;
        scratch_ptr[device] = q;
    }
    *p = scratch_ptr[device];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_build_index_noalloc(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K,
                                              int32_t E, int32_t capacity, int32_t group_size, int32_t alignment,
                                              const moe_index *out, hipStream_t stream)
{
    using namespace moe;
    // every argument error first, before any HIP call
    moe_status st = build_index_impl(topk_idx, topk_w, T, K, E, capacity, group_size, alignment, out, nullptr, 0,
                                     stream, false);
    if (st != MOE_OK)
        return st;
    const Plan p = make_plan(T, K, E, group_size > 0 ? E / group_size : 0);
    if (p.ws > kScratchBytes)
        return MOE_ERR_UNSUPPORTED;  // beyond the scratch's size (no valid input gets here)
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess)
        return MOE_ERR_HIP;
    hipDevice_t stream_device = -1;
    if (hipStreamGetDevice(stream, &stream_device) != hipSuccess)
        return MOE_ERR_HIP;
    if (stream_device != device)
        return MOE_ERR_INVALID;  // the scratch address is the current device's
    void *ws = nullptr;
    if ((st = scratch_address(device, &ws)) != MOE_OK)
        return st;
    return build_index_impl(topk_idx, topk_w, T, K, E, capacity, group_size, alignment, out, ws, kScratchBytes,
                            stream);
}
