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
// store cannot be waited for without waiting for the store too). Three launches, plus one in
// group mode:
//   1. hist   one workgroup per tile of whole tokens: the tile's expert histogram (and the
//             group histogram of each token's first slot in a group) with LDS atomics -- only
//             counts come from atomics, never positions, so the result is deterministic -- and
//             one coalesced row hist[tile][0..E) per tile.
//   2. scan   one workgroup: lanes own 4 consecutive keys, wavefronts own ranges of tiles; the
//             per-wave partial sums meet in LDS, giving each (tile, key) its first row inside
//             the key; a block scan over the key totals gives each key's first row. Also
//             counts, group_list and the capacity bookkeeping.
//   3. rank   one workgroup per tile, its tokens split over 4 wavefronts (per-wave counts and
//             a prefix over the waves in LDS); each wavefront walks its slots 64 at a time in
//             slot order. Lanes with the same key find each other with one ballot per key bit
//             (a match-any built from ballots); their stable rank is popcount(peers &
//             lanes_below) and the last peer advances the key's running row counter in LDS.
//             The workgroups then write the padding or unused rows together.
//   4. esrc   (group mode) expert-major row -> group slot.
// The drop-and-pad capacity rule ([Scratch] §18, §26.6), the expert alignment ([Combine] §6:
// segments rounded up to a multiple of A with padding rows, the segment starts being the scan of
// the aligned lengths) and the group (send once per rank) slots ([CANN] §1(1)) are applied
// inside the same passes. Rows after the last segment are unused slack (MOE_ROW_UNUSED).
#include <algorithm>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMaxTiles = 128;      // tiles grow with T so that there are never more
constexpr int kScanThreads = 1024;  // the scan workgroup: 16 wavefronts
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kKeysPerChunk = 4 * kWave;                                  // 4 keys per lane
constexpr int kTilesPerWave = (kMaxTiles + kScanWaves - 1) / kScanWaves;  // 8
constexpr int kRankBatch = 8;  // 64-slot groups whose loads a rank wave issues together

struct IndexArgs {
    const int32_t *topk_idx;
    const float *topk_w;
    int64_t T;
    int32_t K, E, cap, gs, G;
    int32_t align;   // expert alignment (1: none)
    int32_t Ep, Gp;  // row strides of the histograms (E, G rounded up to a multiple of 4)
    int32_t tile_tokens, ntiles;
    int32_t ebits, gbits;
    int32_t *hist_e;  // [ntiles][Ep] tile counts -> first row of (tile, expert) inside the expert
    int32_t *hist_g;  // [ntiles][Gp] the same for group slots
    int32_t *seg_e;   // [E] first row of each expert
    int32_t *seg_g;   // [G] first slot of each group
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

// ---------------------------------------------------------------- 1. per-tile histograms
__global__ __launch_bounds__(256) void hist_kernel(IndexArgs a)
{
    extern __shared__ int32_t sh[];
    int32_t *he = sh;         // [Ep]
    int32_t *hg = sh + a.Ep;  // [Gp]
    const int tile = blockIdx.x;
    const int nsh = a.Ep + (a.gs > 0 ? a.Gp : 0);
    for (int i = threadIdx.x; i < nsh; i += blockDim.x)
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
    int32_t *row = a.hist_e + static_cast<int64_t>(tile) * a.Ep;
    for (int e = threadIdx.x; e < a.Ep; e += blockDim.x)
        row[e] = he[e];
    if (a.gs > 0) {
        int32_t *rowg = a.hist_g + static_cast<int64_t>(tile) * a.Gp;
        for (int g = threadIdx.x; g < a.Gp; g += blockDim.x)
            rowg[g] = hg[g];
    }
}

// ---------------------------------------------------------------- 2. scan
struct ScanShared {
    int32_t part[kScanWaves][kKeysPerChunk];  // per-wave partial sums -> per-wave prefixes
    int32_t tot[MOE_MAX_EXPERTS];
    int32_t seg[MOE_MAX_EXPERTS];
    int32_t waves[kWave + 1];
};

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

// Exclusive scan of one value per thread over the workgroup; *total gets the sum.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t *sh_waves, int32_t *total)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1)
        sh_waves[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const int32_t w = lane < kScanWaves ? sh_waves[lane] : 0;
        const int32_t winc = wave_inclusive_scan(w);
        if (lane < kScanWaves)
            sh_waves[lane] = winc - w;
        if (lane == kScanWaves - 1)
            sh_waves[kWave] = winc;
    }
    __syncthreads();
    const int32_t r = sh_waves[wave] + inc - v;
    *total = sh_waves[kWave];
    __syncthreads();
    return r;
}

// hist [ntiles][stride] (stride a multiple of 4, 16-byte aligned rows) holds tile counts; on
// return it holds, for every (tile, key), the first row of that tile inside the key, sh.tot the
// key totals and sh.seg each key's first row, the keys' segments being their totals rounded up
// to a multiple of `align`. Returns the grand total of the segments.
__device__ __forceinline__ int32_t scan_tiles(int32_t *hist, int nkeys, int stride, int ntiles, int align,
                                              ScanShared &sh)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int tpw = (ntiles + kScanWaves - 1) / kScanWaves;  // <= kTilesPerWave
    const int j0 = wave * tpw;
    for (int kc = 0; kc < nkeys; kc += kKeysPerChunk) {
        const int key = kc + 4 * lane;  // this lane's 4 keys: key .. key+3
        const bool mine = key < stride;
        u32x4 c[kTilesPerWave];
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            const int tile = j0 + j;
            c[j] = (j < tpw && tile < ntiles && mine) ? ld16(hist + static_cast<int64_t>(tile) * stride + key)
                                                      : u32x4{0u, 0u, 0u, 0u};
        }
        u32x4 s{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            s.x += c[j].x;
            s.y += c[j].y;
            s.z += c[j].z;
            s.w += c[j].w;
        }
        sh.part[wave][4 * lane + 0] = static_cast<int32_t>(s.x);
        sh.part[wave][4 * lane + 1] = static_cast<int32_t>(s.y);
        sh.part[wave][4 * lane + 2] = static_cast<int32_t>(s.z);
        sh.part[wave][4 * lane + 3] = static_cast<int32_t>(s.w);
        __syncthreads();
        if (threadIdx.x < kKeysPerChunk) {  // one thread per key: prefix over the waves
            int32_t run = 0;
            for (int w = 0; w < kScanWaves; ++w) {
                const int32_t v = sh.part[w][threadIdx.x];
                sh.part[w][threadIdx.x] = run;
                run += v;
            }
            if (kc + static_cast<int>(threadIdx.x) < nkeys)
                sh.tot[kc + threadIdx.x] = run;
        }
        __syncthreads();
        u32x4 run{static_cast<uint32_t>(sh.part[wave][4 * lane + 0]), static_cast<uint32_t>(sh.part[wave][4 * lane + 1]),
                  static_cast<uint32_t>(sh.part[wave][4 * lane + 2]), static_cast<uint32_t>(sh.part[wave][4 * lane + 3])};
#pragma unroll
        for (int j = 0; j < kTilesPerWave; ++j) {
            const int tile = j0 + j;
            if (j < tpw && tile < ntiles && mine)
                st16(hist + static_cast<int64_t>(tile) * stride + key, run);
            run.x += c[j].x;
            run.y += c[j].y;
            run.z += c[j].z;
            run.w += c[j].w;
        }
        __syncthreads();  // sh.part is reused by the next chunk of keys
    }
    int32_t total;
    const int32_t v = static_cast<int>(threadIdx.x) < nkeys ? static_cast<int32_t>(round_up(sh.tot[threadIdx.x], align)) : 0;
    const int32_t ex = block_exclusive_scan(v, sh.waves, &total);
    if (static_cast<int>(threadIdx.x) < nkeys)
        sh.seg[threadIdx.x] = ex;
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(IndexArgs a)
{
    __shared__ ScanShared sh;
    const int tid = threadIdx.x;
    const int64_t R = index_rows(a.T, a.K, a.E, a.cap, a.align);
    scan_tiles(a.hist_e, a.E, a.Ep, a.ntiles, a.cap > 0 ? 1 : a.align, sh);
    for (int e = tid; e < a.E; e += kScanThreads) {
        const int32_t cnt = sh.tot[e];
        const int32_t start = sh.seg[e];
        a.seg_e[e] = start;
        a.ix.counts[e] = cnt;
        a.ix.group_list[e] = start + (a.cap > 0 ? cnt : static_cast<int32_t>(round_up(cnt, a.align)));
        if (a.ix.kept_counts)
            a.ix.kept_counts[e] = a.cap > 0 ? min(cnt, a.cap) : cnt;
    }
    if (a.ntiles == 0) {
        // no tokens (otherwise the rank kernel writes these rows): every row of every expert is
        // padding in drop-and-pad, every row is unused slack otherwise
        const int32_t mark = a.cap > 0 ? MOE_ROW_PAD : MOE_ROW_UNUSED;
        for (int64_t r = tid; r < R; r += kScanThreads) {
            a.ix.sorted_indices[r] = mark;
            if (a.ix.permuted_probs)
                a.ix.permuted_probs[r] = 0.0f;
            if (a.gs > 0)
                a.ix.esrc[r] = mark;
        }
    }
    if (a.gs > 0) {
        __syncthreads();  // sh is reused for the group keys
        const int32_t m = scan_tiles(a.hist_g, a.G, a.Gp, a.ntiles, 1, sh);
        for (int g = tid; g < a.G; g += kScanThreads) {
            a.seg_g[g] = sh.seg[g];
            a.ix.group_counts[g] = sh.tot[g];
        }
        if (tid == 0)
            a.ix.n_slots[0] = m;
    }
}

// ---------------------------------------------------------------- 3. stable ranks
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

constexpr int kRankWaves = 4;  // a tile's tokens are split across 4 wavefronts
constexpr int kRankThreads = kRankWaves * kWave;
constexpr int kSpan = kRankBatch * kWave;  // slots whose loads a wavefront issues together

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

__device__ __forceinline__ void load_batch(const IndexArgs &a, int64_t base0, int64_t s1, bool want_w,
                                           int (&e)[kRankBatch], float (&w)[kRankBatch])
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) {
        const int64_t i = base0 + b * kWave + lane;
        e[b] = i < s1 ? a.topk_idx[i] : -1;
        w[b] = want_w && i < s1 ? a.topk_w[i] : 1.0f;
    }
}

// One workgroup per tile, kRankWaves wavefronts, each owning a contiguous quarter of the tile's
// tokens (whole tokens). Phase A: every wave counts its slots per expert (and its first-in-group
// slots per group) in LDS. Phase B: per key, a prefix over the waves starting at the tile's
// first row of the key. Phase C: every wave walks its slots in order, 64 at a time, and ranks
// them against its own running counters. Finally the workgroups together write the padding
// (drop-and-pad) or unused rows.
__global__ __launch_bounds__(kRankThreads) void rank_kernel(IndexArgs a)
{
    extern __shared__ int32_t sh[];
    int32_t *cnt_e = sh;                        // [kRankWaves][E] counts -> next row of the wave
    int32_t *cnt_g = cnt_e + kRankWaves * a.E;  // [kRankWaves][G]
    int32_t *seg_e = cnt_g + kRankWaves * a.G;  // [E] first row of each expert
    int32_t *ids_all = seg_e + a.E;             // [kRankWaves][kSpan] expert ids of each wave's batch
    const int tile = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    int32_t *cw_e = cnt_e + wave * a.E;
    int32_t *cw_g = cnt_g + wave * a.G;
    int32_t *ids = ids_all + wave * kSpan;
    for (int i = tid; i < kRankWaves * (a.E + a.G); i += kRankThreads)
        sh[i] = 0;
    for (int e = tid; e < a.E; e += kRankThreads)
        seg_e[e] = a.seg_e[e];

    // this wave's tokens and slots
    const int64_t tile_t0 = static_cast<int64_t>(tile) * a.tile_tokens;
    const int64_t tile_t1 = min(a.T, tile_t0 + a.tile_tokens);
    const int64_t per = (a.tile_tokens + kRankWaves - 1) / kRankWaves;
    const int64_t t0 = min(tile_t1, tile_t0 + wave * per);
    const int64_t t1 = min(tile_t1, t0 + per);
    const int64_t s0 = t0 * a.K, s1 = t1 * a.K;
    const bool want_w = a.ix.permuted_probs && a.topk_w;
    int e_first[kRankBatch];
    float w_first[kRankBatch];
    load_batch(a, s0, s1, want_w, e_first, w_first);
    __syncthreads();

    // ---- phase A: per-wave counts
    for (int64_t base0 = s0; base0 < s1; base0 += kSpan) {
        int e_b[kRankBatch];
        float w_b[kRankBatch];
        if (base0 == s0) {
#pragma unroll
            for (int b = 0; b < kRankBatch; ++b)
                e_b[b] = e_first[b];
        } else {
            load_batch(a, base0, s1, false, e_b, w_b);
        }
        if (a.gs > 0) {
#pragma unroll
            for (int b = 0; b < kRankBatch; ++b)
                ids[b * kWave + lane] = e_b[b];
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int b = 0; b < kRankBatch; ++b) {
            const int64_t i = base0 + b * kWave + lane;
            const int e = e_b[b];
            if (i >= s1 || !valid_expert(e, a.E))
                continue;
            atomicAdd(&cw_e[e], 1);
            if (a.gs > 0) {
                const int64_t t = i / a.K;
                const int k = static_cast<int>(i - t * a.K);
                const int g = e / a.gs;
                if (first_in_group(a, i, k, g, base0, ids))
                    atomicAdd(&cw_g[g], 1);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // ---- phase B: each wave's first row per key
    {
        const int32_t *hrow = a.hist_e + static_cast<int64_t>(tile) * a.Ep;
        for (int e = tid; e < a.E; e += kRankThreads) {
            int32_t run = seg_e[e] + hrow[e];
            for (int w = 0; w < kRankWaves; ++w) {
                const int32_t c = cnt_e[w * a.E + e];
                cnt_e[w * a.E + e] = run;
                run += c;
            }
        }
        if (a.gs > 0) {
            const int32_t *hrowg = a.hist_g + static_cast<int64_t>(tile) * a.Gp;
            for (int g = tid; g < a.G; g += kRankThreads) {
                int32_t run = a.seg_g[g] + hrowg[g];
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
    int e_nx[kRankBatch];
    float w_nx[kRankBatch];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) {
        e_nx[b] = e_first[b];
        w_nx[b] = w_first[b];
    }
    for (int64_t base0 = s0; base0 < s1; base0 += kSpan) {
        int e_cur[kRankBatch];
        float w_cur[kRankBatch];
#pragma unroll
        for (int b = 0; b < kRankBatch; ++b) {
            e_cur[b] = e_nx[b];
            w_cur[b] = w_nx[b];
        }
        if (base0 + kSpan < s1)  // next batch in flight, issued before this batch's stores
            load_batch(a, base0 + kSpan, s1, want_w, e_nx, w_nx);
        if (a.gs > 0) {
#pragma unroll
            for (int b = 0; b < kRankBatch; ++b)
                ids[b * kWave + lane] = e_cur[b];
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int b = 0; b < kRankBatch; ++b) {
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
            if (a.gs > 0) {
                const int g = ok ? e / a.gs : -1;
                const bool lead = ok && first_in_group(a, i, k, g, base0, ids);
                const uint64_t pg = match_peers(g, a.gbits, __ballot(lead));
                int32_t slot = -1;
                if (lead)
                    slot = cw_g[g] + __popcll(pg & below);
                __builtin_amdgcn_wave_barrier();
                if (lead && lane == last_lane(pg))
                    cw_g[g] += __popcll(pg);
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
    __syncthreads();
    int32_t *cnt = cnt_e;  // reused: per-expert counts
    for (int e = tid; e < a.E; e += kRankThreads)
        cnt[e] = a.ix.counts[e];
    __syncthreads();
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
                    if (a.gs > 0)
                        a.ix.esrc[r] = MOE_ROW_PAD;
                }
            }
        }
        const int64_t total = static_cast<int64_t>(seg_e[a.E - 1]) + round_up(cnt[a.E - 1], A);
        const int64_t R = index_rows(a.T, a.K, a.E, 0, A);
        for (int64_t r = total + static_cast<int64_t>(tile) * kRankThreads + tid; r < R; r += stride) {
            a.ix.sorted_indices[r] = MOE_ROW_UNUSED;
            if (a.ix.permuted_probs)
                a.ix.permuted_probs[r] = 0.0f;
            if (a.gs > 0)
                a.ix.esrc[r] = MOE_ROW_UNUSED;
        }
    }
}

// ---------------------------------------------------------------- 4. group mode: esrc
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

int round4(int n) { return (n + 3) & ~3; }

struct Plan {
    int32_t tile_tokens, ntiles;
    size_t ws_hist_e, ws_e;  // bytes of the expert tile counts, and of those plus the expert starts
    size_t ws_hist_g, ws_g;  // the same for groups
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
    p.ws_hist_e = al(sizeof(int32_t) * static_cast<size_t>(round4(E)) * p.ntiles);
    p.ws_e = p.ws_hist_e + al(sizeof(int32_t) * static_cast<size_t>(E));
    p.ws_hist_g = G > 0 ? al(sizeof(int32_t) * static_cast<size_t>(round4(G)) * p.ntiles) : 0;
    p.ws_g = G > 0 ? p.ws_hist_g + al(sizeof(int32_t) * static_cast<size_t>(G)) : 0;
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

extern "C" int64_t moe_index_rows(int64_t T, int32_t K, int32_t E, int32_t capacity, int32_t alignment)
{
    using namespace moe;
    if (T < 0 || K < 1 || E < 1 || alignment < 0 || (capacity > 0 && alignment > 1))
        return -1;
    const int64_t R = index_rows(T, K, E, capacity > 0 ? capacity : 0, alignment > 1 ? alignment : 1);
    return R > 0x7fffffffLL ? -1 : R;
}

extern "C" moe_status moe_build_index(const int32_t *topk_idx, const float *topk_w, int64_t T,
                                      int32_t K, int32_t E, int32_t capacity, int32_t group_size,
                                      int32_t alignment, const moe_index *out, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream)
{
    using namespace moe;
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
    const Plan p = make_plan(T, K, E, G);
    if (p.ntiles > kMaxTiles)
        return MOE_ERR_UNSUPPORTED;  // cannot happen: tiles grow with T to stay within the limit
    if (!workspace || workspace_bytes < p.ws_e + p.ws_g || !aligned16(workspace))
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
    a.tile_tokens = p.tile_tokens;
    a.ntiles = p.ntiles;
    a.ebits = bits_for(E);
    a.gbits = bits_for(G);
    char *ws = static_cast<char *>(workspace);
    a.hist_e = reinterpret_cast<int32_t *>(ws);
    a.seg_e = reinterpret_cast<int32_t *>(ws + p.ws_hist_e);
    a.hist_g = G > 0 ? reinterpret_cast<int32_t *>(ws + p.ws_e) : nullptr;
    a.seg_g = G > 0 ? reinterpret_cast<int32_t *>(ws + p.ws_e + p.ws_hist_g) : nullptr;
    a.ix = *out;

    if (T == 0) {
        // nothing routed: the scan alone writes zero counts and the padding rows
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
        return launch_status();
    }

    const size_t lds_hist = sizeof(int32_t) * (static_cast<size_t>(a.Ep) + (G > 0 ? a.Gp : 0));
    hipLaunchKernelGGL(hist_kernel, dim3(p.ntiles), dim3(256), lds_hist, stream, a);
    if ((st = launch_status()) != MOE_OK)
        return st;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a);
    if ((st = launch_status()) != MOE_OK)
        return st;
    const size_t lds_rank =
        sizeof(int32_t) * (static_cast<size_t>(kRankWaves) * (E + G) + E + static_cast<size_t>(kRankWaves) * kSpan);
    hipLaunchKernelGGL(rank_kernel, dim3(p.ntiles), dim3(kRankThreads), lds_rank, stream, a);
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
