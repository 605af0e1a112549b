// Row gather: dst[i] = src[src_row[i]] bit for bit, a zero row when src_row[i] is out of range.
// [Megatron] §1.1 step 5 (permuted_input = tokens.index_select(0, sorted_indices));
// [Scratch] §12 (permuted_tokens = tokens[permute_indices]); padded expert buffers are zero
// ([Scratch] §18 drop-and-pad).
//
// Pure HBM traffic. Two forms with identical results:
//   moe_permute          gather: one wavefront per destination row, 16-byte accesses (1 KiB per
//                        wave instruction), kUnroll loads in flight per lane. A source row that
//                        several destinations name is read again for each of them.
//   moe_permute_scatter  source-major: one wavefront per (source row, 1 KiB slice) reads it once
//                        and writes it to all its destinations (the inverse map, e.g. row_of),
//                        so x is read once instead of K times; zero rows come from the gather map.
//   moe_permute_grouped  the gather's map, worked through in groups of destination rows (e.g.
//                        row_of, one group per token): a source row that several rows of one
//                        group name is read once for all of them. The receive side of the group
//                        dispatch uses it: a group slot feeds up to group_size expert rows.
// Destination rows are written with agent-scope streaming stores (see kPolicyStreamStore). Rows
// whose size is not a multiple of 16 bytes (or unaligned bases) take element-wise paths.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts, one row each

// A gather-map entry that asks for a zero row: outside [0, src_rows), but not the unused slack
// after the last segment (MOE_ROW_UNUSED), which no permute writes.
__device__ __forceinline__ bool zero_entry(int32_t s, int64_t src_rows)
{
    return (s < 0 || s >= src_rows) && s != MOE_ROW_UNUSED;
}
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kRowsPerBlock *kWave) void permute_vec16_kernel(
    const char *__restrict__ src, int64_t src_rows, int64_t nvec, const int32_t *__restrict__ src_row,
    int64_t N, char *__restrict__ dst)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock +
                      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    if (i >= N)
        return;
    const int32_t s = src_row[i];
    if (s == MOE_ROW_UNUSED)
        return;
    const int64_t row_bytes = nvec * 16;
    const __amdgpu_buffer_rsrc_t d = make_rsrc(dst + i * row_bytes, static_cast<uint32_t>(row_bytes));
    if (s < 0 || s >= src_rows) {
        const u32x4 z{0u, 0u, 0u, 0u};
        for (int64_t v = lane; v < nvec; v += kWave)
            st16_buf<kPolicyStreamStore>(d, static_cast<uint32_t>(v * 16), z);
        return;
    }
    const char *p = src + static_cast<int64_t>(s) * row_bytes;
    int64_t v = lane;
    for (; v + (kUnroll - 1) * kWave < nvec; v += kUnroll * kWave) {
        u32x4 r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            r[u] = ld16(p + (v + u * kWave) * 16);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            st16_buf<kPolicyStreamStore>(d, static_cast<uint32_t>((v + u * kWave) * 16), r[u]);
    }
    for (; v < nvec; v += kWave)
        st16_buf<kPolicyStreamStore>(d, static_cast<uint32_t>(v * 16), ld16(p + v * 16));
}

template <typename T>
__global__ __launch_bounds__(kRowsPerBlock *kWave) void permute_elem_kernel(
    const T *__restrict__ src, int64_t src_rows, int64_t H, const int32_t *__restrict__ src_row,
    int64_t N, T *__restrict__ dst)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x / kWave);
    if (i >= N)
        return;
    const int32_t s = src_row[i];
    if (s == MOE_ROW_UNUSED)
        return;
    T *d = dst + i * H;
    if (s < 0 || s >= src_rows) {
        for (int64_t h = lane; h < H; h += kWave)
            d[h] = T(0);
        return;
    }
    const T *p = src + static_cast<int64_t>(s) * H;
    for (int64_t h = lane; h < H; h += kWave)
        d[h] = p[h];
}

// ---------------------------------------------------------------- source-major form
// One wavefront per (source row, 1 KiB slice of it) -- two with a dense map, each taking half of
// the destinations (see kScatterParts) --: each lane loads one 16-byte vector of the row and
// stores it to the wave's destinations; the destinations sit in lanes 0..63 (64 entries of dst_of
// at a time; the row is loaded when the wave's first valid one turns up) and are walked in lane
// order with readlane, so the loop is uniform. Other waves write the zero rows:
// each checks `zr` entries of src_row and zero-fills those outside [0, src_rows). Measured at
// T16384 H7168 K8 bf16: 339 us per launch (6.2 TB/s) with slices, 350 us with one 256-thread
// workgroup per row. When the output has more rows than the map can name (N > src_rows * J:
// drop-and-pad, aligned experts) padding is certain and its waves come first, so that they
// overlap the copies instead of trailing them (drop-and-pad at T8192 H4096 E128: 134 -> 125 us),
// 4 rows each (with caches flushed there, 72% of the rows being padding: 129.5 us against 132.5
// with 8 rows per wave, 134.6 with 2, 140.2 with 1 and 143.5 with 16; nontemporal instead of
// sc1|nt zero stores 138.3 us); otherwise they come last, 16 rows each (putting them first cost
// the unpadded case ~1%).
constexpr int kScatterThreads = 256;  // element-wise kernels
constexpr int kScatterWaves = kScatterThreads / kWave;
// workgroups of the 16-byte scatter: 8 wavefronts. The waves of a source row are ordered (half of
// the destinations, slice), so that a workgroup writes up to 8 KiB contiguous to each destination
// of its half. Measured with caches flushed at T16384 H7168 K8 bf16: 364 us against 379 us with
// 4-wave workgroups ordered (slice, half) and 367 / 404 us with 16 / 12 waves; 395 us with 4-wave
// workgroups of 128 threads. Blocks stay in the default round-robin over the XCDs: giving each
// XCD one contiguous range of blocks made this permute 417 us (and drop-and-pad, whose padding
// waves then fell on one XCD, 366 against 140 us).
constexpr int kScatterVecThreads = 512;
constexpr int kScatterVecWaves = kScatterVecThreads / kWave;
// 16-byte vectors of a source row per lane of a scatter wavefront: at T16384 H7168 K8 bf16 one
// (1 KiB per wavefront) took 342 us, two 348 us and four 355 us; 128- or 512-thread workgroups
// changed nothing at that size and lost at drop-and-pad T8192 H4096 E128 (128: 134 against 125 us)
constexpr int kScatterVecs = 1;
constexpr int kZeroRowsPerWave = 16;
constexpr int kZeroRowsPerWaveFirst = 4;
// Waves per (source row, slice). With a dense map -- one output row per map entry, as the standard
// dispatch's row_of is -- every row has J destinations, and two waves per slice each store to half
// of them: wave p takes the valid destinations ranked [4p, 4p + 4) in column order, the last wave
// the rest. On MI355X a wave's first stores are the cheap ones (8 GiB of 1 KiB stores ran at 7.1
// TB/s with one store per wave, 5.7-6.1 TB/s with 2-16; fanned out 1 KiB -> 8 destinations at 5.8
// TB/s with 2-4 stores per wave, 5.45 TB/s with 8, 4.7 TB/s with 1): at T16384 H7168 K8 bf16 the
// permute took 379 us instead of 395 us with caches flushed. Sparse maps (the group send's 32
// columns with ~3 destinations, drop-and-pad rows with ~3 of 8 kept) keep one wave per slice: there
// the second wave mostly finds nothing to store (drop-and-pad 140 -> 147 us, group send 78 -> 98 us);
// so did three or four waves per slice on the dense map (473 and 485 us: each loads the slice).
constexpr int kScatterDestsPerWave = 4;
constexpr int kScatterParts = 2;
inline int scatter_parts(int J, int64_t src_rows, int64_t N)
{
    return J > kScatterDestsPerWave && N == src_rows * J ? kScatterParts : 1;
}
// Paired order (two parts): the workgroups come in blocks of 2 x 8; workgroup j < 8 of a block takes
// part 0 and workgroup j + 8 part 1 of the same 8 x 8 (source row, slice) pairs. Blocks are dealt
// to the 8 XCDs round-robin, so the two waves that read one slice run at about the same time on
// the same XCD and the second read hits its L2: the PMC fetches of the permute at T16384 H7168 K8
// bf16 fall from 1.11x to 1.00x its algorithmic bytes. It pays only in the weighted scatter (the
// combine backward's dy = w * dout: 358 -> 352 us); the plain copy's time did not follow its
// fetches (358 -> 360 us; 355 -> 365 us once both orders had 32-bit indices), so it keeps the
// (row, part, slice) order. The waves are short (1 KiB
// to at most four rows), so their index arithmetic shows: with 32-bit instead of 64-bit divisions
// the permute took 355 instead of 358 us (T16384 H7168 K8), 133.0 against 133.3 us with padding
// (T8192 H4096 E128) and 74.6 against 75.6 us as the group send.
__host__ __device__ inline int64_t scatter_copy_waves(int64_t units, int parts, bool paired)
{
    return paired ? ceil_div(units, static_cast<int64_t>(kXcds) * kScatterVecWaves) * 2 * kXcds * kScatterVecWaves
                  : units * parts;
}
constexpr int kMaxScatterDests = MOE_MAX_EXPERTS;  // dst_of columns (e.g. one per expert group)
constexpr int kMaxGroupDests = kWave;               // destinations of one group of the grouped gather

// Zero-fills rows first .. first+zr-1 whose src_row entry asks for a zero row (one wavefront;
// no-op without a gather map), and the same rows of the companion rows dst2 (nw2 4-byte words
// each; none when nw2 is 0). zr <= 64.
__device__ __forceinline__ void zero_rows_wave(int64_t src_rows, int64_t nvec, const int32_t *__restrict__ src_row,
                                               int64_t N, int64_t first, char *__restrict__ dst,
                                               int zr = kZeroRowsPerWave, char *__restrict__ dst2 = nullptr,
                                               int nw2 = 0)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row_bytes = nvec * 16;
    const int64_t i = first + lane;
    const bool zero = src_row && lane < zr && i < N && zero_entry(src_row[i], src_rows);
    uint64_t m = __ballot(zero);
    const u32x4 z{0u, 0u, 0u, 0u};
    while (m) {
        const int j = __builtin_ctzll(m);
        m &= m - 1;
        const __amdgpu_buffer_rsrc_t d = make_rsrc(dst + (first + j) * row_bytes, static_cast<uint32_t>(row_bytes));
        for (int64_t v = lane; v < nvec; v += kWave)
            st16_buf<kPolicyStreamStore>(d, static_cast<uint32_t>(v * 16), z);
        if (nw2 > 0) {
            const uint32_t rb2 = static_cast<uint32_t>(nw2) * 4u;
            const __amdgpu_buffer_rsrc_t d2 = make_rsrc(dst2 + (first + j) * static_cast<int64_t>(rb2), rb2);
            for (int w = lane; w < nw2; w += kWave)
                __builtin_amdgcn_raw_buffer_store_b32(0u, d2, w * 4, 0, kPolicyStreamStore);
        }
    }
}

// SCALE: bf16 rows, destination j of source row t receives scale[t*J + j] * row (float32
// products, rounded to bf16 to nearest even): the backward of the weighted combine, dy = w * dout.
template <bool SCALE>
__global__ __launch_bounds__(kScatterVecThreads) void permute_scatter_vec16_kernel(
    const char *__restrict__ src, int64_t src_rows, int64_t nvec, const int32_t *__restrict__ dst_of, int J,
    const int32_t *__restrict__ src_row, int64_t N, char *__restrict__ dst, int64_t zero_waves, bool zero_first,
    int parts, bool paired, const float *__restrict__ scale)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row_bytes = nvec * 16;
    // every wave index fits in 32 bits (the launcher refuses grids of 2^31 waves or more), and
    // 32-bit division is far cheaper than 64-bit for these short-lived waves
    const uint32_t spr = static_cast<uint32_t>((nvec + kWave * kScatterVecs - 1) / (kWave * kScatterVecs));
    const uint32_t wpr = spr * static_cast<uint32_t>(parts);
    const uint32_t gw = blockIdx.x * kScatterVecWaves +
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave)));
    const uint32_t units = static_cast<uint32_t>(src_rows) * spr;  // (source row, slice) pairs
    const uint32_t copy_waves = static_cast<uint32_t>(scatter_copy_waves(units, parts, paired));
    const uint32_t zwaves = static_cast<uint32_t>(zero_waves);
    // wave index -> zero window or copy wave; the grid's last workgroup may hold up to 7 waves
    // past both (zero windows past N check nothing, copy rows past src_rows return below)
    const uint32_t zw = zero_first ? gw : gw - copy_waves;
    if (zero_first ? gw < zwaves : gw >= copy_waves) {
        const int zr = zero_first ? kZeroRowsPerWaveFirst : kZeroRowsPerWave;
        zero_rows_wave(src_rows, nvec, src_row, N, static_cast<int64_t>(zw) * zr, dst, zr);
        return;
    }
    const uint32_t cw = zero_first ? gw - zwaves : gw;
    int part;
    int64_t t, slice;
    if (paired) {  // (two parts, so no leading zero waves: cw starts at a workgroup)
        const uint32_t cb = cw / kScatterVecWaves;
        const uint32_t sb = cb / (2 * kXcds);
        const uint32_t j = cb % (2 * kXcds);
        part = static_cast<int>(j / kXcds);
        const uint32_t u = (sb * kXcds + j % kXcds) * kScatterVecWaves + cw % kScatterVecWaves;
        if (u >= units)
            return;
        const uint32_t t32 = u / spr;
        t = t32;
        slice = u - t32 * spr;
    } else {  // waves of a row: (part, slice); at most two parts
        const uint32_t t32 = cw / wpr;
        if (t32 >= static_cast<uint32_t>(src_rows))
            return;
        const uint32_t rem = cw - t32 * wpr;
        part = rem >= spr ? 1 : 0;
        t = t32;
        slice = rem - static_cast<uint32_t>(part) * spr;
    }
    const int64_t v0 = slice * kWave * kScatterVecs + lane;  // this lane's first vector of the row
    // this wave's share: the row's valid destinations ranked [lo, hi) in column order
    const int lo = part * kScatterDestsPerWave;
    const int hi = part == parts - 1 ? 0x7fffffff : lo + kScatterDestsPerWave;
    u32x4 r[kScatterVecs];
    bool loaded = false;  // wave-uniform
    // loads the slice on first use, then stores it (scaled by ws of lane j for SCALE) to row `row`
    auto store_to = [&](int32_t row, float ws, int j) {
        if (!loaded) {
#pragma unroll
            for (int i = 0; i < kScatterVecs; ++i) {
                const int64_t v = v0 + i * kWave;
                r[i] = u32x4{0u, 0u, 0u, 0u};
                if (v < nvec)
                    r[i] = ld16(src + t * row_bytes + v * 16);
            }
            loaded = true;
        }
        const __amdgpu_buffer_rsrc_t q =
            make_rsrc(dst + static_cast<int64_t>(row) * row_bytes, static_cast<uint32_t>(row_bytes));
#pragma unroll
        for (int i = 0; i < kScatterVecs; ++i) {
            const int64_t v = v0 + i * kWave;
            u32x4 o = r[i];
            if constexpr (SCALE) {
                const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ws), j));
                o = u32x4{pack_bf16x2(wj * bf16_lo(r[i].x), wj * bf16_hi(r[i].x)),
                          pack_bf16x2(wj * bf16_lo(r[i].y), wj * bf16_hi(r[i].y)),
                          pack_bf16x2(wj * bf16_lo(r[i].z), wj * bf16_hi(r[i].z)),
                          pack_bf16x2(wj * bf16_lo(r[i].w), wj * bf16_hi(r[i].w))};
            }
            if (v < nvec)
                st16_buf<kPolicyStreamStore>(q, static_cast<uint32_t>(v * 16), o);
        }
    };
    if (SCALE && parts > 1 && J <= kWave) {
        // weighted scatter over two waves: the row's valid destinations are split by address, wave
        // p taking those ranked [4p, 4p + 4) by destination row (ties by column, the last wave the
        // rest), and each wave stores in ascending row order. At T16384 H7168 K8 bf16 the combine
        // backward took 600 instead of 631 us (both halves sorted ascending or both descending
        // measured alike; column-order halves were the 631 us), in group mode 309 instead of 320 us;
        // the plain copy measured no faster with the same split (360.5 against 359.0 us)
        const int32_t my = lane < J ? dst_of[t * J + lane] : -1;
        const float ws = lane < J && scale ? scale[t * J + lane] : 1.0f;
        const bool valid = my >= 0 && my < N;
        const uint64_t m = __ballot(valid);
        int rank = 0;  // valid lanes before this one in (row, column) order
        for (uint64_t mm = m; mm;) {
            const int j = __builtin_ctzll(mm);
            mm &= mm - 1;
            const int32_t dj = __builtin_amdgcn_readlane(my, j);
            rank += (dj < my || (dj == my && j < lane)) ? 1 : 0;
        }
        for (int rk = lo; rk < hi; ++rk) {
            const uint64_t b = __ballot(valid && rank == rk);
            if (!b)
                break;
            const int j = __builtin_ctzll(b);
            store_to(__builtin_amdgcn_readlane(my, j), ws, j);
        }
        return;
    }
    int seen = 0;                                        // valid destinations before this chunk
    for (int j0 = 0; j0 < J && seen < hi; j0 += kWave) {  // the destinations, 64 entries at a time
        const int32_t my = j0 + lane < J ? dst_of[t * J + j0 + lane] : -1;
        float ws = 1.0f;
        if constexpr (SCALE)
            ws = j0 + lane < J && scale ? scale[t * J + j0 + lane] : 1.0f;  // loaded beside the destination
        uint64_t m = __ballot(my >= 0 && my < N);
        const int nm = __popcll(m);
        if (seen + nm <= lo) {
            seen += nm;
            continue;
        }
        for (; seen < lo; ++seen)  // the valid destinations of the previous waves' shares
            m &= m - 1;
        for (; m && seen < hi; ++seen) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            store_to(__builtin_amdgcn_readlane(my, j), ws, j);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kScatterThreads) void permute_scatter_elem_kernel(
    const T *__restrict__ src, int64_t src_rows, int64_t H, const int32_t *__restrict__ dst_of, int J,
    const int32_t *__restrict__ src_row, int64_t N, T *__restrict__ dst)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (static_cast<int64_t>(blockIdx.x) >= src_rows) {
        const int64_t first = (static_cast<int64_t>(blockIdx.x) - src_rows) * (kScatterThreads / kWave) * kZeroRowsPerWave +
                              static_cast<int64_t>(threadIdx.x / kWave) * kZeroRowsPerWave;
        const int64_t i = first + lane;
        const bool zero = lane < kZeroRowsPerWave && i < N && zero_entry(src_row[i], src_rows);
        uint64_t m = __ballot(zero);
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            T *d = dst + (first + j) * H;
            for (int64_t h = lane; h < H; h += kWave)
                d[h] = T(0);
        }
        return;
    }
    const int64_t t = blockIdx.x;
    const T *p = src + t * H;
    for (int j0 = 0; j0 < J; j0 += kWave) {  // every wave walks the same entries
        const int32_t my = j0 + lane < J ? dst_of[t * J + j0 + lane] : -1;
        uint64_t m = __ballot(my >= 0 && my < N);
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            T *q = dst + static_cast<int64_t>(__builtin_amdgcn_readlane(my, j)) * H;
            for (int64_t h = threadIdx.x; h < H; h += kScatterThreads)
                q[h] = p[h];
        }
    }
}

// ---------------------------------------------------------------- grouped gather
// One wavefront per (group of destination rows, 1 KiB slice) -- two for groups of more than four
// rows, each taking half of them (see kScatterParts) --: lanes 0..J-1 hold the group's
// destination rows and their source rows (src_of beside them when the caller has it, else
// src_row[d] one dependent load later). The distinct source rows are taken kGroupLoads at a
// time: their slices are loaded first (all in flight together; gfx9 completes vector-memory
// operations in order, so a load issued after a store would wait for it), then stored to every
// destination of the wave's share that names them. Waves past the last group write the zero
// rows, as in the source-major form. The element-wise form looks sources up through src_row
// (src_of, when given, names the same rows).
constexpr int kGroupLoads = 4;
// workgroups of the grouped gather: 2 wavefronts (at T8192 H7168 with 32 groups of 8: 241 us
// against 245 us with 4)
constexpr int kGroupedThreads = 128;
constexpr int kGroupedWaves = kGroupedThreads / kWave;
constexpr int kGroupLoadPolicy = 0;

// Companion rows (the FP8 scales of moe_permute_grouped_fp8): words [0, nw2) of row s of src2
// go to row d of dst2 for every destination of the wave's share (mask m over the lanes holding
// d and their source sr), one source at a time. Taken by the waves of a group's first slice.
__device__ __forceinline__ void grouped_companion(const char *__restrict__ src2, char *__restrict__ dst2, int nw2,
                                                  int32_t sr, int32_t d, uint64_t m)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t rb2 = static_cast<uint32_t>(nw2) * 4u;
    while (m) {
        const int32_t s = __builtin_amdgcn_readlane(sr, __builtin_ctzll(m));
        const uint64_t p0 = __ballot(sr == s) & m;
        m &= ~p0;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(src2 + static_cast<int64_t>(s) * rb2, rb2);
        for (int w = lane; w < nw2; w += kWave) {
            const uint32_t v = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, w * 4, 0, 0));
            uint64_t p = p0;
            while (p) {
                const int j = __builtin_ctzll(p);
                p &= p - 1;
                const __amdgpu_buffer_rsrc_t q =
                    make_rsrc(dst2 + static_cast<int64_t>(__builtin_amdgcn_readlane(d, j)) * rb2, rb2);
                __builtin_amdgcn_raw_buffer_store_b32(v, q, w * 4, 0, kPolicyStreamStore);
            }
        }
    }
}

// COMP: the companion rows are moved too (moe_permute_grouped_fp8); the plain gather's instance
// carries none of their code.
template <bool COMP>
__global__ __launch_bounds__(kGroupedThreads) void permute_grouped_vec16_kernel(
    const char *__restrict__ src, int64_t src_rows, int64_t nvec, const int32_t *__restrict__ src_row,
    const int32_t *__restrict__ dst_of, int64_t M, int J, int64_t N, const int32_t *__restrict__ src_of,
    char *__restrict__ dst, int parts, const char *__restrict__ src2, char *__restrict__ dst2, int nw2)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row_bytes = nvec * 16;
    const int64_t wpr = (nvec + kWave - 1) / kWave * parts;  // waves per group of destination rows
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * kGroupedWaves +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int64_t copy_waves = M * wpr;
    if (gw >= copy_waves) {
        zero_rows_wave(src_rows, nvec, src_row, N, (gw - copy_waves) * kZeroRowsPerWave, dst, kZeroRowsPerWave,
                       dst2, COMP ? nw2 : 0);
        return;
    }
    const int64_t g = gw / wpr;
    const int64_t rem = gw - g * wpr;
    const int part = static_cast<int>(rem % parts);
    const int64_t v = (rem / parts) * kWave + lane;
    const int32_t d = lane < J ? dst_of[g * J + lane] : -1;
    // the source of each destination: given beside it (both loads in flight together), or looked
    // up through the gather map once the destination is known
    const int32_t so = src_of && lane < J ? src_of[g * J + lane] : -1;
    const bool dv = d >= 0 && d < N;
    const int32_t sr = src_of ? (dv ? so : -1) : (dv ? src_row[d] : -1);
    const bool ok = dv && sr >= 0 && sr < src_rows;
    uint64_t m = __ballot(ok);
    // this wave's share of the group's rows: ranks [4 part, 4 part + 4) in lane order, the last
    // wave the rest (see kScatterParts)
    for (int i = 0; i < part * kScatterDestsPerWave && m; ++i)
        m &= m - 1;
    if (part != parts - 1) {
        uint64_t keep = 0;
        for (int i = 0; i < kScatterDestsPerWave && m; ++i) {
            keep |= m & (~m + 1);
            m &= m - 1;
        }
        m = keep;
    }
    // the first slice's waves also move the companion rows: up to 64 words with the slice's own
    // loads and stores (one word per lane), longer rows in a pass of their own first
    const bool comp = COMP && nw2 > 0 && rem < parts;
    const bool comp_inline = comp && nw2 <= kWave;
    if (comp && !comp_inline)
        grouped_companion(src2, dst2, nw2, sr, d, m);
    const uint32_t rb2 = static_cast<uint32_t>(nw2) * 4u;
    while (m) {
        int32_t sb[kGroupLoads];
        uint64_t pb[kGroupLoads];
#pragma unroll
        for (int u = 0; u < kGroupLoads; ++u) {
            sb[u] = -1;
            pb[u] = 0;
            if (m) {
                sb[u] = __builtin_amdgcn_readlane(sr, __builtin_ctzll(m));
                pb[u] = __ballot(sr == sb[u]) & m;  // lanes naming this source (valid ones only)
                m &= ~pb[u];
            }
        }
        // unguarded loads (an absent source has a zero-size resource, a lane past the row reads
        // beyond the resource's end: both read zeros), then one wait for all of them, so that the
        // stores below issue back to back: with a guarded load per source the compiler could not
        // count the loads and waited for all earlier stores before each source's stores
        u32x4 r[kGroupLoads];
        uint32_t c2[kGroupLoads];
#pragma unroll
        for (int u = 0; u < kGroupLoads; ++u) {
            const __amdgpu_buffer_rsrc_t s = make_rsrc(src + static_cast<int64_t>(sb[u] < 0 ? 0 : sb[u]) * row_bytes,
                                                       sb[u] < 0 ? 0u : static_cast<uint32_t>(row_bytes));
            r[u] = ld16_buf<kGroupLoadPolicy>(s, static_cast<uint32_t>(v * 16));
            c2[u] = 0u;
            if (comp_inline) {  // lanes past the row read zeros (the resource's bound)
                const __amdgpu_buffer_rsrc_t s2 =
                    make_rsrc(src2 + static_cast<int64_t>(sb[u] < 0 ? 0 : sb[u]) * rb2, sb[u] < 0 ? 0u : rb2);
                c2[u] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(s2, lane * 4, 0, 0));
            }
        }
        // the loaded values pass through an empty asm statement: it keeps every load ahead of the
        // first store (the compiler may not sink one into the store loop) and puts the one wait here
#pragma unroll
        for (int u = 0; u < kGroupLoads; ++u)
            asm volatile("" : : "v"(r[u].x), "v"(r[u].y), "v"(r[u].z), "v"(r[u].w), "v"(c2[u]));
#pragma unroll
        for (int u = 0; u < kGroupLoads; ++u) {
            uint64_t p = pb[u];
            while (p) {
                const int j = __builtin_ctzll(p);
                p &= p - 1;
                const int32_t dj = __builtin_amdgcn_readlane(d, j);
                const __amdgpu_buffer_rsrc_t q =
                    make_rsrc(dst + static_cast<int64_t>(dj) * row_bytes, static_cast<uint32_t>(row_bytes));
                if (v < nvec)
                    st16_buf<kPolicyStreamStore>(q, static_cast<uint32_t>(v * 16), r[u]);
                if (comp_inline && lane < nw2)
                    __builtin_amdgcn_raw_buffer_store_b32(c2[u], make_rsrc(dst2 + static_cast<int64_t>(dj) * rb2, rb2),
                                                          lane * 4, 0, kPolicyStreamStore);
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kScatterThreads) void permute_grouped_elem_kernel(
    const T *__restrict__ src, int64_t src_rows, int64_t H, const int32_t *__restrict__ src_row,
    const int32_t *__restrict__ dst_of, int64_t M, int J, int64_t N, T *__restrict__ dst)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (static_cast<int64_t>(blockIdx.x) >= M) {
        const int64_t first = (static_cast<int64_t>(blockIdx.x) - M) * kScatterWaves * kZeroRowsPerWave +
                              static_cast<int64_t>(threadIdx.x / kWave) * kZeroRowsPerWave;
        const int64_t i = first + lane;
        const bool zero = lane < kZeroRowsPerWave && i < N && zero_entry(src_row[i], src_rows);
        uint64_t m = __ballot(zero);
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            T *q = dst + (first + j) * H;
            for (int64_t h = lane; h < H; h += kWave)
                q[h] = T(0);
        }
        return;
    }
    const int64_t g = blockIdx.x;
    for (int j0 = 0; j0 < J; j0 += kWave) {  // every wave walks the same entries
        const int j = j0 + lane;
        const int32_t d = j < J ? dst_of[g * J + j] : -1;
        const bool dv = d >= 0 && d < N;
        const int32_t sr = dv ? src_row[d] : -1;
        uint64_t m = __ballot(dv && sr >= 0 && sr < src_rows);
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const T *p = src + static_cast<int64_t>(__builtin_amdgcn_readlane(sr, k)) * H;
            T *q = dst + static_cast<int64_t>(__builtin_amdgcn_readlane(d, k)) * H;
            for (int64_t h = threadIdx.x; h < H; h += kScatterThreads)
                q[h] = p[h];
        }
    }
}

}  // namespace

moe_status launch_scatter_vec16(const char *src, int64_t src_rows, int64_t nvec, const int32_t *dst_of, int J,
                                const int32_t *src_row, int64_t N, char *dst, bool scaled, const float *scale,
                                hipStream_t stream)
{
    const bool zero_first = src_row && N > src_rows * J;  // padding rows are certain
    const int64_t zwaves = src_row ? ceil_div(N, zero_first ? kZeroRowsPerWaveFirst : kZeroRowsPerWave) : 0;
    const int parts = scatter_parts(J, src_rows, N);
    const int64_t units = src_rows * ceil_div(nvec, static_cast<int64_t>(kWave) * kScatterVecs);
    const bool paired = scaled && parts == kScatterParts;
    const int64_t waves = scatter_copy_waves(units, parts, paired) + zwaves;
    const int64_t blocks = ceil_div(waves, kScatterVecWaves);
    if (blocks * kScatterVecWaves > 0x7fffffff)  // the kernel's wave indices are 32-bit
        return MOE_ERR_UNSUPPORTED;
    if (blocks == 0)
        return MOE_OK;
    if (scaled)
        hipLaunchKernelGGL(permute_scatter_vec16_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kScatterVecThreads),
                           0, stream, src, src_rows, nvec, dst_of, J, src_row, N, dst, zwaves, zero_first, parts, paired, scale);
    else
        hipLaunchKernelGGL(permute_scatter_vec16_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                           dim3(kScatterVecThreads), 0, stream, src, src_rows, nvec, dst_of, J, src_row, N, dst, zwaves,
                           zero_first, parts, paired, nullptr);
    return launch_status();
}

}  // namespace moe

extern "C" moe_status moe_permute_scatter(const void *src, int64_t src_rows, int64_t H, moe_dtype dt,
                                          const int32_t *dst_of, int32_t J, const int32_t *src_row, int64_t N,
                                          void *dst, hipStream_t stream)
{
    using namespace moe;
    if (src_rows < 0 || H < 1 || N < 0 || J < 1 || (dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_FP8_E4M3))
        return MOE_ERR_INVALID;
    if (J > kMaxScatterDests)
        return MOE_ERR_UNSUPPORTED;
    if (N == 0 || (src_rows == 0 && !src_row))
        return MOE_OK;
    if (!dst || (src_rows > 0 && (!src || !dst_of)))
        return MOE_ERR_INVALID;
    const int64_t esz = dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1);
    const int64_t row_bytes = H * esz;
    if (row_bytes > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    const int64_t zero_waves = src_row ? ceil_div(N, kZeroRowsPerWave) : 0;
    if (row_bytes % 16 == 0 && aligned16(dst) && (src_rows == 0 || aligned16(src)))
        return launch_scatter_vec16(static_cast<const char *>(src), src_rows, row_bytes / 16, dst_of, J, src_row, N,
                                    static_cast<char *>(dst), false, nullptr, stream);
    const int64_t blocks = src_rows + ceil_div(zero_waves, kScatterWaves);
    if (blocks > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kScatterThreads);
    if (esz == 4) {
        hipLaunchKernelGGL(permute_scatter_elem_kernel<uint32_t>, grid, block, 0, stream,
                           static_cast<const uint32_t *>(src), src_rows, H, dst_of, J, src_row, N,
                           static_cast<uint32_t *>(dst));
    } else if (esz == 2) {
        hipLaunchKernelGGL(permute_scatter_elem_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t *>(src), src_rows, H, dst_of, J, src_row, N,
                           static_cast<uint16_t *>(dst));
    } else {
        hipLaunchKernelGGL(permute_scatter_elem_kernel<uint8_t>, grid, block, 0, stream,
                           static_cast<const uint8_t *>(src), src_rows, H, dst_of, J, src_row, N,
                           static_cast<uint8_t *>(dst));
    }
    return launch_status();
}

extern "C" moe_status moe_permute(const void *src, int64_t src_rows, int64_t H, moe_dtype dt,
                                  const int32_t *src_row, int64_t N, void *dst, hipStream_t stream)
{
    using namespace moe;
    if (src_rows < 0 || H < 1 || N < 0 || (dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_FP8_E4M3))
        return MOE_ERR_INVALID;
    if (N == 0)
        return MOE_OK;
    if (!src_row || !dst || (src_rows > 0 && !src))
        return MOE_ERR_INVALID;
    const int64_t blocks = ceil_div(N, kRowsPerBlock);
    const int64_t esz = dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1);
    const int64_t row_bytes = H * esz;
    if (blocks > 0x7fffffff || row_bytes > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kRowsPerBlock * kWave);
    if (row_bytes % 16 == 0 && aligned16(dst) && (src_rows == 0 || aligned16(src))) {
        hipLaunchKernelGGL(permute_vec16_kernel, grid, block, 0, stream, static_cast<const char *>(src),
                           src_rows, row_bytes / 16, src_row, N, static_cast<char *>(dst));
    } else if (esz == 4) {
        hipLaunchKernelGGL(permute_elem_kernel<uint32_t>, grid, block, 0, stream,
                           static_cast<const uint32_t *>(src), src_rows, H, src_row, N,
                           static_cast<uint32_t *>(dst));
    } else if (esz == 2) {
        hipLaunchKernelGGL(permute_elem_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t *>(src), src_rows, H, src_row, N,
                           static_cast<uint16_t *>(dst));
    } else {
        hipLaunchKernelGGL(permute_elem_kernel<uint8_t>, grid, block, 0, stream,
                           static_cast<const uint8_t *>(src), src_rows, H, src_row, N,
                           static_cast<uint8_t *>(dst));
    }
    return launch_status();
}

namespace moe {
namespace {
// moe_permute_grouped, with companion rows (nw2 > 0: float32 rows of nw2 values, moved to the same
// destinations from the same sources, zeroed with the same zero rows) for moe_permute_grouped_fp8.
moe_status launch_grouped(const void *src, int64_t src_rows, int64_t H, moe_dtype dt, const int32_t *src_row,
                          int64_t N, const int32_t *dst_of, int64_t M, int32_t J, const int32_t *src_of, void *dst,
                          const float *src2, float *dst2, int64_t nw2, hipStream_t stream)
{
    if (src_rows < 0 || H < 1 || N < 0 || M < 0 || J < 1 || (dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_FP8_E4M3))
        return MOE_ERR_INVALID;
    if (J > kMaxGroupDests)
        return MOE_ERR_UNSUPPORTED;
    if (N == 0)
        return MOE_OK;
    if (!src_row || !dst || (M > 0 && !dst_of) || (src_rows > 0 && !src))
        return MOE_ERR_INVALID;
    if (nw2 > 0 && (!dst2 || (src_rows > 0 && !src2)))
        return MOE_ERR_INVALID;
    const int64_t esz = dt == MOE_F32 ? 4 : (dt == MOE_BF16 ? 2 : 1);
    const int64_t row_bytes = H * esz;
    if (row_bytes > 0x7fffffffLL || nw2 * 4 > 0x7fffffffLL)
        return MOE_ERR_UNSUPPORTED;
    const int64_t zero_waves = ceil_div(N, kZeroRowsPerWave);
    if (row_bytes % 16 == 0 && aligned16(dst) && (src_rows == 0 || aligned16(src))) {
        const int64_t nvec = row_bytes / 16;
        // two waves per slice, each storing to half of a group's rows, for groups of more than
        // four rows of at least one full slice: at T8192 H7168 (32 groups of 8) 233 -> 225 us,
        // FP8 codes 120 -> 118 us; the 224-byte rows of FP8 scales lost (11.8 -> 15.6 us)
        const int parts = J > kScatterDestsPerWave && nvec >= kWave ? kScatterParts : 1;
        const int64_t blocks = ceil_div(M * ceil_div(nvec, kWave) * parts + zero_waves, kGroupedWaves);
        if (blocks > 0x7fffffff)
            return MOE_ERR_UNSUPPORTED;
        if (nw2 > 0)
            hipLaunchKernelGGL(permute_grouped_vec16_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                               dim3(kGroupedThreads), 0, stream, static_cast<const char *>(src), src_rows, nvec,
                               src_row, dst_of, M, J, N, src_of, static_cast<char *>(dst), parts,
                               reinterpret_cast<const char *>(src2), reinterpret_cast<char *>(dst2),
                               static_cast<int>(nw2));
        else
            hipLaunchKernelGGL(permute_grouped_vec16_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                               dim3(kGroupedThreads), 0, stream, static_cast<const char *>(src), src_rows, nvec,
                               src_row, dst_of, M, J, N, src_of, static_cast<char *>(dst), parts, nullptr, nullptr, 0);
        return launch_status();
    }
    const int64_t blocks = M + ceil_div(zero_waves, kScatterWaves);
    if (blocks > 0x7fffffff)
        return MOE_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kScatterThreads);
    if (esz == 4) {
        hipLaunchKernelGGL(permute_grouped_elem_kernel<uint32_t>, grid, block, 0, stream,
                           static_cast<const uint32_t *>(src), src_rows, H, src_row, dst_of, M, J, N,
                           static_cast<uint32_t *>(dst));
    } else if (esz == 2) {
        hipLaunchKernelGGL(permute_grouped_elem_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t *>(src), src_rows, H, src_row, dst_of, M, J, N,
                           static_cast<uint16_t *>(dst));
    } else {
        hipLaunchKernelGGL(permute_grouped_elem_kernel<uint8_t>, grid, block, 0, stream,
                           static_cast<const uint8_t *>(src), src_rows, H, src_row, dst_of, M, J, N,
                           static_cast<uint8_t *>(dst));
    }
    const moe_status st = launch_status();
    if (st != MOE_OK || nw2 == 0)
        return st;
    // rows without 16-byte vectors: the companion rows by a second element-wise pass
    return launch_grouped(src2, src_rows, nw2, MOE_F32, src_row, N, dst_of, M, J, src_of, dst2, nullptr, nullptr, 0,
                          stream);
}
}  // namespace
}  // namespace moe

extern "C" moe_status moe_permute_grouped(const void *src, int64_t src_rows, int64_t H, moe_dtype dt,
                                          const int32_t *src_row, int64_t N, const int32_t *dst_of, int64_t M,
                                          int32_t J, const int32_t *src_of, void *dst, hipStream_t stream)
{
    return moe::launch_grouped(src, src_rows, H, dt, src_row, N, dst_of, M, J, src_of, dst, nullptr, nullptr, 0,
                               stream);
}

extern "C" moe_status moe_permute_grouped_fp8(const uint8_t *src, const float *src_scales, int64_t src_rows,
                                              int64_t H, int32_t block, const int32_t *src_row, int64_t N,
                                              const int32_t *dst_of, int64_t M, int32_t J, const int32_t *src_of,
                                              uint8_t *dst, float *dst_scales, hipStream_t stream)
{
    if (block < 1 || H < 1 || H % block != 0)
        return MOE_ERR_INVALID;
    return moe::launch_grouped(src, src_rows, H, MOE_FP8_E4M3, src_row, N, dst_of, M, J, src_of, dst, src_scales,
                               dst_scales, H / block, stream);
}
