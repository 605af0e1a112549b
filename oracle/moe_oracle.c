/*
 * moe_oracle.c -- plain, slow CPU oracle for the MoE token dispatch / unpermute-combine path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's CPU-baseline leg
 * may load or call this library. The product path (the HIP library and its Python binding)
 * never does, and this file shares no code, header, table or constant with it.
 *
 * Every function follows a passage of the source pages, cited by page title and section:
 *   [Combine]   "03 · Combine 与 forward / backward 对称性" (llm-infra-atlas, EP chapter)
 *   [Scratch]   "从零理解 MoE 算子：路由、专家并行与 Token 重排" (171host)
 *   [CANN]      CANN Dispatch&Combine optimisation notes (cann.csdn.net), "Dispatch&Combine优化"
 *   [Megatron]  "token dispatcher + fuse_a2a" (obnotes, Megatron/transformer-moe)
 *
 * Conventions (shared with the HIP path only by documentation, never by code):
 *   - row-major, contiguous arrays; all indices and counts int32; weights float32;
 *   - a top-k slot whose expert id is outside [0, E) (the pages' "no expert", written -1)
 *     routes nowhere; a row index outside the valid range selects nothing (a zero row in a
 *     permute, a skipped term in a combine);
 *   - dtype codes: 0 = float32, 1 = bf16 (raw uint16 bits); FP8 E4M3 codes are raw bytes (the
 *     permute copies rows of 1, 2 or 4 bytes per element).
 * Return codes: 0 ok, 1 invalid argument, 2 unsupported combination.
 *
 * Parity status: every function here is pinned by the CPU tests (worked examples printed on
 * the pages, closed forms, invariants, brute force, exact error bounds).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC -lm
 * (no contraction, so every multiply-add below is exactly the one written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_INVALID 1
#define ORC_UNSUPPORTED 2

/* ---------------------------------------------------------------- number formats ---- */

/* bf16 -> float32: the bf16 bits are the upper half of the float32 bits (exact). */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN of the same sign. */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

static float load_elem(const void *base, int dt, int64_t i)
{
    if (dt == 0)
        return ((const float *)base)[i];
    return bf16_to_f32(((const uint16_t *)base)[i]);
}

static void store_elem(void *base, int dt, int64_t i, float v)
{
    if (dt == 0)
        ((float *)base)[i] = v;
    else
        ((uint16_t *)base)[i] = f32_to_bf16(v);
}

uint16_t oracle_f32_to_bf16(float f) { return f32_to_bf16(f); }

/* FP8 E4M3 (the OCP 8-bit format, "fn": no infinities): 1 sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; 0x7f / 0xff are NaN, so the
 * largest finite magnitude is 0x7e = 1.75 * 2^8 = 448. Rounding to nearest, ties to even; a
 * magnitude that rounds above 448 saturates to 448 (the conversion used for the dispatch). */
static uint8_t f32_to_e4m3(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if (isnan(f))
        return (uint8_t)(sign | 0x7f);
    double a = fabs((double)f);
    if (a > 448.0)                     /* rounds to 448 or beyond it: saturates (infinity too) */
        return (uint8_t)(sign | 0x7e);
    if (a < 0x1p-6) {                 /* subnormal range: a multiple of 2^-9 */
        double m = nearbyint(a * 512.0); /* exact scaling; default rounding: ties to even */
        return (uint8_t)(sign | (uint8_t)m); /* m == 8 is the smallest normal, code 0x08 */
    }
    int ex;
    double fr = frexp(a, &ex);          /* a = fr * 2^ex, fr in [0.5, 1) */
    int E = ex - 1;                     /* a = (1 + t) * 2^E */
    double mant = nearbyint((a / ldexp(1.0, E) - 1.0) * 8.0);
    (void)fr;
    if (mant == 8.0) {
        mant = 0.0;
        E += 1;
    }
    return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | (int)mant));
}

static float e4m3_to_f32(uint8_t c)
{
    int sign = c & 0x80, E = (c >> 3) & 15, m = c & 7;
    double v;
    if (E == 15 && m == 7)
        v = NAN;
    else if (E == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, E - 7);
    return (float)(sign ? -v : v);
}

uint8_t oracle_f32_to_e4m3(float f) { return f32_to_e4m3(f); }
float oracle_e4m3_to_f32(uint8_t c) { return e4m3_to_f32(c); }

/* ---------------------------------------------------------------- capacity ---------- */

/* [Scratch] §18: expert_capacity = ceil(tokens * top_k / num_experts * capacity_factor).
 * The capacity factor is passed as the exact fraction cf_num/cf_den and the ceiling is taken
 * in integers, so 1024 tokens, top_k 2, 8 experts, factor 1.25 give 256 * 1.25 = 320. */
int64_t oracle_capacity(int64_t tokens, int32_t top_k, int32_t num_experts,
                        int32_t cf_num, int32_t cf_den)
{
    if (tokens < 0 || top_k < 1 || num_experts < 1 || cf_num < 0 || cf_den < 1)
        return -1;
    int64_t num = tokens * (int64_t)top_k * (int64_t)cf_num;
    int64_t den = (int64_t)num_experts * (int64_t)cf_den;
    return (num + den - 1) / den;
}

/* ---------------------------------------------------------------- routing ----------- */

/* [Scratch] §3 (and the same two lines in §27): the K experts with the largest router
 * logits are selected (topk), then the weights are a softmax over those K scores only.
 * Reading of the open points:
 *   - slot k holds the k-th expert in the order (logit descending, expert id ascending):
 *     a tie goes to the lower id, and +0 == -0 is a tie (plain IEEE comparison);
 *   - [Scratch] §26.7 notes the router softmax is precision sensitive, so it is evaluated in
 *     double: w_k = exp(s_k - s_0) / sum_j exp(s_j - s_0) (s_0 is the largest selected logit),
 *     the sum taken in slot order, each weight rounded once to float.
 * Logits must be finite; E >= K. */
/* The K best experts of one token among those not yet taken (taken[e] = 1 excludes e), slot k
 * the k-th in the order (score descending, id ascending), and the softmax over their scores. */
static void select_and_softmax(const float *s, int32_t E, int32_t K, unsigned char *taken, int32_t *idx,
                               double *ex, float *w)
{
    for (int32_t k = 0; k < K; ++k) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || s[e] > s[best]) /* strict: an equal score keeps the lower id */
                best = e;
        }
        taken[best] = 1;
        idx[k] = best;
    }
    double m = (double)s[idx[0]];
    double z = 0.0;
    for (int32_t k = 0; k < K; ++k) {
        ex[k] = exp((double)s[idx[k]] - m);
        z += ex[k];
    }
    for (int32_t k = 0; k < K; ++k)
        w[k] = (float)(ex[k] / z);
}

int oracle_route_topk(const float *logits, int64_t T, int32_t E, int32_t K,
                      int32_t *topk_idx, float *topk_w)
{
    if (T < 0 || E < 1 || K < 1 || K > E || (T > 0 && (!logits || !topk_idx || !topk_w)))
        return ORC_INVALID;
    unsigned char *taken = malloc((size_t)E);
    double *ex = malloc(sizeof(double) * (size_t)K);
    if (!taken || !ex) {
        free(taken);
        free(ex);
        return ORC_INVALID;
    }
    for (int64_t t = 0; t < T; ++t) {
        memset(taken, 0, (size_t)E);
        select_and_softmax(logits + t * E, E, K, taken, topk_idx + t * K, ex, topk_w + t * K);
    }
    free(taken);
    free(ex);
    return ORC_OK;
}

/* Group-limited routing, [Scratch] §21: the experts are split into groups (here contiguous,
 * g = e / group_size), the router first picks a few groups and then the top experts inside
 * them, so that a token's experts sit in at most topk_groups groups (ranks).
 * Reading of the open points (the page defines no group score):
 *   - a group's score is the largest logit among its experts (so topk_groups = G is plain
 *     routing, and the token's best expert is always kept);
 *   - the topk_groups groups with the largest scores are taken, an equal score going to the
 *     lower group id (+0 == -0 a tie);
 *   - the K experts and their weights are then chosen exactly as in oracle_route_topk, among
 *     the experts of the chosen groups only.
 * Requires group_size dividing E, 1 <= topk_groups <= G and K <= topk_groups * group_size. */
int oracle_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t K, int32_t group_size,
                              int32_t topk_groups, int32_t *topk_idx, float *topk_w)
{
    if (T < 0 || E < 1 || K < 1 || K > E || group_size < 1 || E % group_size != 0 || topk_groups < 1 ||
        topk_groups > E / group_size || (int64_t)K > (int64_t)topk_groups * group_size ||
        (T > 0 && (!logits || !topk_idx || !topk_w)))
        return ORC_INVALID;
    int32_t G = E / group_size;
    unsigned char *taken = malloc((size_t)E);
    unsigned char *chosen = malloc((size_t)G);
    float *score = malloc(sizeof(float) * (size_t)G);
    double *ex = malloc(sizeof(double) * (size_t)K);
    if (!taken || !chosen || !score || !ex) {
        free(taken);
        free(chosen);
        free(score);
        free(ex);
        return ORC_INVALID;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *s = logits + t * E;
        for (int32_t g = 0; g < G; ++g) {
            int32_t top = g * group_size;
            for (int32_t e = g * group_size; e < (g + 1) * group_size; ++e)
                if (s[e] > s[top])
                    top = e;
            score[g] = s[top];
        }
        memset(chosen, 0, (size_t)G);
        for (int32_t m = 0; m < topk_groups; ++m) {
            int32_t bg = -1;
            for (int32_t g = 0; g < G; ++g) {
                if (chosen[g])
                    continue;
                if (bg < 0 || score[g] > score[bg])
                    bg = g;
            }
            chosen[bg] = 1;
        }
        for (int32_t e = 0; e < E; ++e)
            taken[e] = chosen[e / group_size] ? 0 : 1;
        select_and_softmax(s, E, K, taken, topk_idx + t * K, ex, topk_w + t * K);
    }
    free(taken);
    free(chosen);
    free(score);
    free(ex);
    return ORC_OK;
}

/* ---------------------------------------------------------------- index build ------- */

/* The expert-major index, following [Megatron] §1.1 (the permute() walk-through):
 *   1. routing_map [tokens, experts] marks which expert each token chose; it is transposed to
 *      [experts, tokens];
 *   2./3. a token-id matrix of the same shape is masked with it; masked_select scans row by
 *      row, so the result lists, expert by expert, the tokens routed there in ascending order:
 *      that list is sorted_indices, and position r in it is the expert-major row r;
 *   4. the router probabilities are transposed and masked the same way: permuted_probs.
 * Here the map is kept as [experts][tokens][K] (slot k remembered), scanned in that order,
 * which equals the pages' walk when a token's experts are distinct and orders repeated
 * experts by slot. Derived outputs:
 *   counts[e]      number of rows of expert e ([Megatron] §1.2 "num_tokens_per_expert");
 *   group_list[e]  inclusive running sum of counts ([Scratch] §7: [3,2,4] -> [3,5,9], expert e
 *                  owns rows [group_list[e]-counts[e], group_list[e]));
 *   row_of[t,k]    the row that slot (t,k) went to, i.e. the saved permute index that makes
 *                  the mapping invertible ([Scratch] §16, §26.5); -1 when the slot routes
 *                  nowhere.
 * Drop-and-pad (capacity > 0), [Scratch] §18 and §26.6: expert e owns the fixed rows
 * [e*cap, (e+1)*cap); the p-th token of expert e in the scan (p from 0) is kept at row
 * e*cap + p when p < cap and dropped otherwise (row_of = -1, it adds nothing in the combine);
 * rows past min(counts[e], cap) are padding: sorted_indices = -1, permuted_probs = 0.
 * kept_counts[e] = min(counts[e], cap).
 * Expert alignment (alignment A > 1, no capacity), [Combine] §6 (dispatch(..., expert_alignment=
 * 128)) and the per-expert receive counts that DeepEP aligns before publishing them: expert e's
 * segment is rounded up to ceil(counts[e]/A)*A rows, its tokens first (in the same order), then
 * padding rows (sorted_indices = -1, permuted_probs = 0); group_list is the running sum of the
 * aligned lengths, so every segment starts at a multiple of A. The buffer holds
 * R = T*K + E*(A-1) rows, the most the aligned segments can need.
 * Rows after the last segment (in the aligned layout, or when slots route nowhere) are unused
 * slack: sorted_indices = -2, permuted_probs = 0 (no permute writes them).
 * Group mode (group_size > 0), [CANN] §1(1): experts form contiguous groups
 * g = e / group_size (a group stands for a rank); a token is sent once per group it uses.
 * The group slots are listed group by group, tokens ascending, in gsrc; slot_of[t,g] is the
 * slot of (t,g) or -1; n_slots = number of slots; esrc[r] is the group slot that feeds
 * expert-major row r (the copy inside the group to each expert's input).
 * Drop-and-pad together with group mode is not supported. */
int oracle_build_index(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K,
                       int32_t E, int32_t capacity, int32_t group_size, int32_t alignment,
                       int32_t *counts, int32_t *group_list, int32_t *kept_counts,
                       int32_t *sorted_indices, int32_t *row_of, float *permuted_probs,
                       int32_t *slot_of, int32_t *gsrc, int32_t *esrc, int32_t *group_counts,
                       int32_t *n_slots, int32_t *slot_src)
{
    if (T < 0 || K < 1 || E < 1 || !counts || !group_list || !sorted_indices || !row_of ||
        (T > 0 && !topk_idx))
        return ORC_INVALID;
    if (capacity > 0 && (group_size > 0 || alignment > 1))
        return ORC_UNSUPPORTED;
    int64_t A = alignment > 1 ? alignment : 1;
    int64_t R = capacity > 0 ? (int64_t)E * capacity : T * K + (int64_t)E * (A - 1);
    if (group_size > 0 && (E % group_size != 0 || !slot_of || !gsrc || !esrc ||
                           !group_counts || !n_slots))
        return ORC_INVALID;

    for (int64_t i = 0; i < T * K; ++i)
        row_of[i] = -1;

    /* masked_select over the [E][T][K] map, row-major */
    int64_t r = 0;
    for (int32_t e = 0; e < E; ++e) {
        int64_t start = r;
        int64_t p = 0; /* position inside expert e's segment */
        for (int64_t t = 0; t < T; ++t) {
            for (int32_t k = 0; k < K; ++k) {
                if (topk_idx[t * K + k] != e)
                    continue;
                if (capacity > 0) {
                    if (p < capacity) {
                        int64_t row = (int64_t)e * capacity + p;
                        sorted_indices[row] = (int32_t)t;
                        row_of[t * K + k] = (int32_t)row;
                        if (permuted_probs)
                            permuted_probs[row] = topk_w ? topk_w[t * K + k] : 1.0f;
                    }
                } else {
                    sorted_indices[r] = (int32_t)t;
                    row_of[t * K + k] = (int32_t)r;
                    if (permuted_probs)
                        permuted_probs[r] = topk_w ? topk_w[t * K + k] : 1.0f;
                    r++;
                }
                p++;
            }
        }
        counts[e] = (int32_t)p;
        if (capacity == 0) {
            /* rows up to the aligned end of the segment are padding */
            for (int64_t end = start + (p + A - 1) / A * A; r < end; ++r) {
                sorted_indices[r] = -1;
                if (permuted_probs)
                    permuted_probs[r] = 0.0f;
            }
        }
    }

    int64_t run = 0;
    for (int32_t e = 0; e < E; ++e) {
        run += capacity > 0 ? counts[e] : (counts[e] + A - 1) / A * A;
        group_list[e] = (int32_t)run;
    }

    if (capacity > 0) {
        for (int32_t e = 0; e < E; ++e) {
            int32_t kept = counts[e] < capacity ? counts[e] : capacity;
            if (kept_counts)
                kept_counts[e] = kept;
            for (int32_t p = kept; p < capacity; ++p) {
                int64_t row = (int64_t)e * capacity + p;
                sorted_indices[row] = -1;
                if (permuted_probs)
                    permuted_probs[row] = 0.0f;
            }
        }
    } else {
        if (kept_counts)
            for (int32_t e = 0; e < E; ++e)
                kept_counts[e] = counts[e];
        /* rows after the last segment are unused slack */
        for (int64_t q = r; q < R; ++q) {
            sorted_indices[q] = -2;
            if (permuted_probs)
                permuted_probs[q] = 0.0f;
        }
    }

    if (group_size > 0) {
        int32_t G = E / group_size;
        for (int64_t i = 0; i < T * (int64_t)G; ++i)
            slot_of[i] = -1;
        int64_t m = 0;
        for (int32_t g = 0; g < G; ++g) {
            int64_t cnt = 0;
            for (int64_t t = 0; t < T; ++t) {
                int uses = 0;
                for (int32_t k = 0; k < K; ++k) {
                    int32_t e = topk_idx[t * K + k];
                    if (e >= 0 && e < E && e / group_size == g)
                        uses = 1;
                }
                if (uses) {
                    gsrc[m] = (int32_t)t;
                    slot_of[t * G + g] = (int32_t)m;
                    m++;
                    cnt++;
                }
            }
            group_counts[g] = (int32_t)cnt;
        }
        *n_slots = (int32_t)m;
        /* expert-major row r holds token sorted_indices[r] for expert e(r); padding rows -1,
           unused slack -2 */
        for (int64_t q = 0; q < R; ++q)
            esrc[q] = q < r ? -1 : -2;
        for (int64_t t = 0; t < T; ++t)
            for (int32_t k = 0; k < K; ++k) {
                int32_t e = topk_idx[t * K + k];
                int32_t row = row_of[t * K + k];
                if (e < 0 || e >= E || row < 0)
                    continue;
                esrc[row] = slot_of[t * G + e / group_size];
            }
        /* the same group slot seen from the routing slot: slot (t, k) is fed by the group slot of
           token t and its expert's group, -1 when the slot routes nowhere (may be NULL) */
        if (slot_src)
            for (int64_t t = 0; t < T; ++t)
                for (int32_t k = 0; k < K; ++k) {
                    int32_t e = topk_idx[t * K + k];
                    int32_t row = row_of[t * K + k];
                    slot_src[t * K + k] = (e < 0 || e >= E || row < 0) ? -1 : slot_of[t * G + e / group_size];
                }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------- permute ----------- */

/* [Megatron] §1.1 step 5 (permuted_input = tokens.index_select(0, sorted_indices)) and
 * [Scratch] §12 (permuted_tokens = tokens[permute_indices]): row i of the output is a bitwise
 * copy of source row src_row[i]. A src_row outside [0, src_rows) (the padding rows of the
 * drop-and-pad and aligned layouts carry -1) gives a row of zeros ([Scratch] §18 padded expert
 * buffers); src_row = -2 marks unused slack, a row that is left as it is.
 * elem_bytes is the size of one hidden element (4, 2, or 1 for FP8 codes). */
int oracle_permute(const void *src, int64_t src_rows, int64_t H, int32_t elem_bytes,
                   const int32_t *src_row, int64_t N, void *dst)
{
    if (src_rows < 0 || H < 1 || N < 0 || (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) ||
        (N > 0 && (!src_row || !dst)) || (src_rows > 0 && !src))
        return ORC_INVALID;
    size_t row_bytes = (size_t)H * (size_t)elem_bytes;
    for (int64_t i = 0; i < N; ++i) {
        unsigned char *d = (unsigned char *)dst + (size_t)i * row_bytes;
        int32_t s = src_row[i];
        if (s >= 0 && s < src_rows)
            memcpy(d, (const unsigned char *)src + (size_t)s * row_bytes, row_bytes);
        else if (s != -2)
            memset(d, 0, row_bytes);
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------- combine ----------- */

/* Unpermute + weighted top-k merge. [Combine] §1: out[t] = sum over the token's top-k experts
 * of probs[t,e] * expert_e(x[t]); [Scratch] §16: output[token] = sum_k weight[token,k] *
 * expert_output[token,k], which requires mapping every expert output back to its token and
 * slot -- here row_of[t,k] names the row of y holding expert_output[token,k]
 * ([Scratch] §13: unpermute is the inverse of the permute).
 * Arithmetic, as fixed for this path: float32 accumulator starting at +0, one fused
 * multiply-add per slot in slot order k = 0..K-1, skipping slots whose row is outside
 * [0, y_rows); w == NULL means every weight is 1 (the pure-add combine of [Combine] §2.3/§3).
 * A bias ([Combine] §3: DeepEP's combine adds an optional final bias), an array shaped and typed
 * like the output, is added in float32 after the sum (one addition), before the output is
 * stored as float32 or rounded to bf16 (nearest even). */
int oracle_unpermute_combine(const void *y, int32_t y_dt, int64_t y_rows, int64_t H,
                             const int32_t *row_of, const float *w, const void *bias, int64_t T,
                             int32_t K, void *out, int32_t out_dt)
{
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || (y_dt != 0 && y_dt != 1) ||
        (out_dt != 0 && out_dt != 1) || (T > 0 && (!row_of || !out)) || (y_rows > 0 && !y))
        return ORC_INVALID;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int32_t r = row_of[t * K + k];
                if (r < 0 || r >= y_rows)
                    continue;
                float wk = w ? w[t * K + k] : 1.0f;
                acc = fmaf(wk, load_elem(y, y_dt, (int64_t)r * H + h), acc);
            }
            if (bias)
                acc = acc + load_elem(bias, out_dt, t * H + h);
            store_elem(out, out_dt, t * H + h, acc);
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------- group pre-combine -- */

/* [CANN] §1(2): before results leave a rank, the outputs of a token's experts that live on the
 * same rank are merged locally with their router weights; the partial results are then
 * summed with the other ranks' ones. Here a rank is a contiguous group of group_size experts.
 * For every (t, g) with s = slot_of[t*G + g] in [0, slots_cap):
 *   partials[s] = sum over k with topk_idx[t,k] in group g (and a valid row) of
 *                 w[t,k] * y[row_of[t,k]]   -- float32, fused multiply-add in slot order,
 * an empty sum being +0, stored as float32 (p_dt 0) or rounded once to bf16 (p_dt 1: the
 * partials are what crosses the exchange, and [Combine] §3 has DeepEP's combine send BF16).
 * The final sum over groups is the combine above called with y = partials, row_of = slot_of,
 * w = NULL and K = G (groups in ascending order). */
int oracle_group_precombine(const void *y, int32_t y_dt, int64_t y_rows, int64_t H,
                            const int32_t *row_of, const float *w, const int32_t *topk_idx,
                            int64_t T, int32_t K, int32_t E, int32_t group_size,
                            const int32_t *slot_of, int64_t slots_cap, void *partials, int32_t p_dt)
{
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || E < 1 || group_size < 1 ||
        E % group_size != 0 || (y_dt != 0 && y_dt != 1) || (p_dt != 0 && p_dt != 1) || slots_cap < 0 ||
        (T > 0 && (!row_of || !topk_idx || !slot_of)) || (slots_cap > 0 && !partials) ||
        (y_rows > 0 && !y))
        return ORC_INVALID;
    int32_t G = E / group_size;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t g = 0; g < G; ++g) {
            int32_t s = slot_of[t * G + g];
            if (s < 0 || s >= slots_cap)
                continue;
            for (int64_t h = 0; h < H; ++h) {
                float acc = 0.0f;
                for (int32_t k = 0; k < K; ++k) {
                    int32_t e = topk_idx[t * K + k];
                    int32_t r = row_of[t * K + k];
                    if (e < 0 || e >= E || e / group_size != g || r < 0 || r >= y_rows)
                        continue;
                    float wk = w ? w[t * K + k] : 1.0f;
                    acc = fmaf(wk, load_elem(y, y_dt, (int64_t)r * H + h), acc);
                }
                store_elem(partials, p_dt, (int64_t)s * H + h, acc);
            }
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------- backward ------------ */

/* Backward of the weighted unpermute-combine. [Combine] §4: the path is linear in the expert
 * outputs, so its backward is the transposed map -- the backward of the combine is a dispatch
 * of the output gradient back to the expert rows (§4.1, and the forward/backward table of
 * §4.2) -- and the router gradient reaches only the selected slots (§6, the closing
 * pseudo-code). With the weights applied in the combine, out[t] = sum_k w[t,k] y[row_of[t,k]]:
 *   dy[r, :] = w[t,k] * dout[t, :] for every (t, k) whose r = row_of[t,k] is in [0, y_rows)
 *              (a float32 product, stored as float32 or rounded to bf16); every other row of dy
 *              fed no output and is zero. A row is named by at most one (t, k) (precondition);
 *   dw[t, k] = sum_h dout[t,h] * y[r,h] for a valid r, else 0 -- the dot product summed in
 *              double and rounded once to float32.
 * w == NULL is the pure-add combine: dy[r] = dout[t]. dw may be NULL (not computed). */
int oracle_combine_backward(const void *dout, int32_t dout_dt, const void *y, int32_t y_dt, int64_t y_rows,
                            int64_t H, const int32_t *row_of, const float *w, int64_t T, int32_t K,
                            void *dy, int32_t dy_dt, float *dw)
{
    if (y_rows < 0 || H < 1 || T < 0 || K < 1 || (dout_dt != 0 && dout_dt != 1) || (y_dt != 0 && y_dt != 1) ||
        (dy_dt != 0 && dy_dt != 1) || (T > 0 && (!row_of || !dout)) || (y_rows > 0 && (!dy || (dw && !y))))
        return ORC_INVALID;
    for (int64_t r = 0; r < y_rows; ++r)
        for (int64_t h = 0; h < H; ++h)
            store_elem(dy, dy_dt, r * H + h, 0.0f);
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = row_of[t * K + k];
            if (r < 0 || r >= y_rows) {
                if (dw)
                    dw[t * K + k] = 0.0f;
                continue;
            }
            float wk = w ? w[t * K + k] : 1.0f;
            for (int64_t h = 0; h < H; ++h)
                store_elem(dy, dy_dt, (int64_t)r * H + h, wk * load_elem(dout, dout_dt, t * H + h));
            if (dw) {
                double s = 0.0;
                for (int64_t h = 0; h < H; ++h)
                    s += (double)load_elem(dout, dout_dt, t * H + h) * (double)load_elem(y, y_dt, (int64_t)r * H + h);
                dw[t * K + k] = (float)s;
            }
        }
    }
    return ORC_OK;
}

/* Backward of route_topk's softmax over the K selected logits ([Scratch] §3 and §27: the
 * softmax runs over the selected scores; [Combine] §6: only the selected experts carry router
 * gradient -- the top-k selection itself is piecewise constant). With w = topk_w (the forward's
 * output, all K slots taking part in the softmax) and g = d_topk_w, the softmax Jacobian
 * dw_k/ds_j = w_k (delta_kj - w_j) gives
 *   d_logits[t, topk_idx[t,k]] += w[t,k] * (g[t,k] - sum_j w[t,j] g[t,j])
 * in double, slots in order k = 0..K-1, the sum over j in slot order; each entry is rounded
 * once to float32; logits outside the selection get 0, slots with an id outside [0, E) give
 * nothing. */
int oracle_route_topk_backward(const int32_t *topk_idx, const float *topk_w, const float *d_topk_w, int64_t T,
                               int32_t E, int32_t K, float *d_logits)
{
    if (T < 0 || E < 1 || K < 1 || K > E || (T > 0 && (!topk_idx || !topk_w || !d_topk_w || !d_logits)))
        return ORC_INVALID;
    double *acc = (double *)malloc(sizeof(double) * (size_t)E);
    if (!acc)
        return ORC_INVALID;
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int32_t j = 0; j < K; ++j)
            s += (double)topk_w[t * K + j] * (double)d_topk_w[t * K + j];
        for (int32_t e = 0; e < E; ++e)
            acc[e] = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = topk_idx[t * K + k];
            if (e < 0 || e >= E)
                continue;
            acc[e] += (double)topk_w[t * K + k] * ((double)d_topk_w[t * K + k] - s);
        }
        for (int32_t e = 0; e < E; ++e)
            d_logits[t * E + e] = (float)acc[e];
    }
    free(acc);
    return ORC_OK;
}


/* ---------------------------------------------------------------- FP8 dispatch -------- */

/* FP8 dispatch ([Combine] §3: the dispatch sends FP8 while the combine stays BF16; [Megatron],
 * the DeepEP dispatch call: x travels with x_scales, num_scales scale groups per token along
 * the hidden dimension). Reading: each token's hidden vector is cut into blocks of `block`
 * consecutive elements (block = H: one scale per token); per block
 *   amax  = max |x|,  scale = amax / 448 (float32 division; 1 when amax is 0),
 *   q[i]  = e4m3(x[i] / scale)   (float32 division, then nearest-even E4M3 with saturation),
 * so that x[i] ~ e4m3_value(q[i]) * scale. q is [T, H] bytes, scales [T, H / block] float32.
 * The dispatch then moves q rows and scale rows with the same gather map (oracle_permute with
 * 1-byte and 4-byte elements). Requires block dividing H. */
int oracle_quantize_fp8(const void *x, int32_t x_dt, int64_t T, int64_t H, int32_t block, uint8_t *q,
                        float *scales)
{
    if (T < 0 || H < 1 || block < 1 || H % block != 0 || (x_dt != 0 && x_dt != 1) ||
        (T > 0 && (!x || !q || !scales)))
        return ORC_INVALID;
    int64_t nb = H / block;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < nb; ++b) {
            float amax = 0.0f;
            for (int64_t i = b * block; i < (b + 1) * block; ++i) {
                float a = fabsf(load_elem(x, x_dt, t * H + i));
                if (a > amax)
                    amax = a;
            }
            float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
            scales[t * nb + b] = scale;
            for (int64_t i = b * block; i < (b + 1) * block; ++i)
                q[t * H + i] = f32_to_e4m3(load_elem(x, x_dt, t * H + i) / scale);
        }
    }
    return ORC_OK;
}
