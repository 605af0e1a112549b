/*
 * Memory-safety driver of the CPU oracle (test infrastructure): every oracle function is run over
 * small edge-case shapes -- no tokens, slots that route nowhere, repeated experts, drop-and-pad,
 * expert groups, alignment, float32 and bf16 rows, FP8 blocks, group-limited routing -- on heap
 * buffers of exactly the sizes the calls are documented to touch, so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer stops at the first access outside them.
 * Exit status 0 when every call returned its expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t oracle_capacity(int64_t tokens, int32_t top_k, int32_t num_experts, int32_t cf_num, int32_t cf_den);
int oracle_route_topk(const float *logits, int64_t T, int32_t E, int32_t K, int32_t *idx, float *w);
int oracle_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t K, int32_t group_size,
                              int32_t topk_groups, int32_t *idx, float *w);
int oracle_build_index(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K, int32_t E,
                       int32_t capacity, int32_t group_size, int32_t alignment, int32_t *counts,
                       int32_t *group_list, int32_t *kept_counts, int32_t *sorted_indices, int32_t *row_of,
                       float *permuted_probs, int32_t *slot_of, int32_t *gsrc, int32_t *esrc,
                       int32_t *group_counts, int32_t *n_slots, int32_t *slot_src);
int oracle_permute(const void *src, int64_t src_rows, int64_t H, int32_t elem_bytes, const int32_t *src_row,
                   int64_t N, void *dst);
int oracle_unpermute_combine(const void *y, int32_t y_dt, int64_t y_rows, int64_t H, const int32_t *row_of,
                             const float *w, const void *bias, int64_t T, int32_t K, void *out, int32_t out_dt);
int oracle_group_precombine(const void *y, int32_t y_dt, int64_t y_rows, int64_t H, const int32_t *row_of,
                            const float *w, const int32_t *topk_idx, int64_t T, int32_t K, int32_t E,
                            int32_t group_size, const int32_t *slot_of, int64_t slots_cap, void *partials,
                            int32_t p_dt);
int oracle_combine_backward(const void *dout, int32_t dout_dt, const void *y, int32_t y_dt, int64_t y_rows,
                            int64_t H, const int32_t *row_of, const float *w, int64_t T, int32_t K, void *dy,
                            int32_t dy_dt, float *dw);
int oracle_route_topk_backward(const int32_t *topk_idx, const float *topk_w, const float *d_topk_w, int64_t T,
                               int32_t E, int32_t K, float *d_logits);
int oracle_quantize_fp8(const void *x, int32_t x_dt, int64_t T, int64_t H, int32_t block, uint8_t *q,
                        float *scales);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(rng >> 33);
}
static float next_f(void) { return ((float)(next_u32() % 20001) - 10000.0f) / 2500.0f; }

/* exactly n bytes (at least 1, so that a zero-size buffer is still a distinct allocation) */
static void *xalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    memset(p, 0xA5, n ? n : 1);
    return p;
}

static int failures = 0;
#define EXPECT(cond)                                                                  \
    do {                                                                              \
        if (!(cond)) {                                                                \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                               \
        }                                                                             \
    } while (0)

static void fill_rows(void *a, int dt, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        float f = next_f();
        if (dt == 0) {
            ((float *)a)[i] = f;
        } else {
            uint32_t u;
            memcpy(&u, &f, 4);
            ((uint16_t *)a)[i] = (uint16_t)(u >> 16);
        }
    }
}

static void one_case(int64_t T, int32_t E, int32_t K, int64_t H, int dt, int32_t cap, int32_t gs, int32_t align,
                     int holes, int repeats, int limited)
{
    const int64_t esz = dt == 0 ? 4 : 2;
    const int32_t G = gs > 0 ? E / gs : 0;
    const int64_t A = align > 1 ? align : 1;
    const int64_t R = cap > 0 ? (int64_t)E * cap : T * K + (int64_t)E * (A - 1);

    float *logits = xalloc(sizeof(float) * T * E);
    for (int64_t i = 0; i < T * E; ++i)
        logits[i] = next_f();
    int32_t *idx = xalloc(sizeof(int32_t) * T * K);
    float *w = xalloc(sizeof(float) * T * K);
    if (limited && gs > 0) {
        int32_t m = 1 + (int32_t)(next_u32() % (uint32_t)G);
        while ((int64_t)m * gs < K)
            ++m;
        EXPECT(oracle_route_topk_grouped(logits, T, E, K, gs, m, idx, w) == 0);
    } else {
        EXPECT(oracle_route_topk(logits, T, E, K, idx, w) == 0);
    }
    for (int64_t i = 0; i < T * K; ++i) {
        if (holes && next_u32() % 5 == 0)
            idx[i] = (next_u32() % 2) ? -1 : E + 3; /* routes nowhere */
        if (repeats && i % K == 1)
            idx[i] = idx[i - 1];
    }

    int32_t *counts = xalloc(4 * (size_t)E), *gl = xalloc(4 * (size_t)E), *kept = xalloc(4 * (size_t)E);
    int32_t *si = xalloc(4 * (size_t)R), *row_of = xalloc(4 * (size_t)(T * K));
    float *pp = xalloc(4 * (size_t)R);
    int32_t *slot_of = NULL, *gsrc = NULL, *esrc = NULL, *gcnt = NULL, *nsl = NULL, *ssrc = NULL;
    const int64_t slots = gs > 0 ? T * (K < G ? K : G) : 0;
    if (gs > 0) {
        slot_of = xalloc(4 * (size_t)(T * G));
        gsrc = xalloc(4 * (size_t)slots);
        esrc = xalloc(4 * (size_t)R);
        gcnt = xalloc(4 * (size_t)G);
        nsl = xalloc(4);
        ssrc = xalloc(4 * (size_t)(T * K));
    }
    EXPECT(oracle_build_index(idx, w, T, K, E, cap, gs, align, counts, gl, kept, si, row_of, pp, slot_of, gsrc,
                              esrc, gcnt, nsl, ssrc) == 0);
    const int64_t n = gs > 0 ? *nsl : 0;
    EXPECT(n <= slots);

    void *x = xalloc((size_t)(T * H * esz));
    fill_rows(x, dt, T * H);
    void *xp = xalloc((size_t)(R * H * esz));
    EXPECT(oracle_permute(x, T, H, (int32_t)esz, si, R, xp) == 0);
    if (gs > 0) {
        void *gbuf = xalloc((size_t)(n * H * esz));
        EXPECT(oracle_permute(x, T, H, (int32_t)esz, gsrc, n, gbuf) == 0);
        EXPECT(oracle_permute(gbuf, n, H, (int32_t)esz, esrc, R, xp) == 0);
        free(gbuf);
    }

    void *y = xalloc((size_t)(R * H * esz));
    fill_rows(y, dt, R * H);
    void *bias = xalloc((size_t)(T * H * esz));
    fill_rows(bias, dt, T * H);
    void *out = xalloc((size_t)(T * H * esz));
    EXPECT(oracle_unpermute_combine(y, dt, R, H, row_of, w, NULL, T, K, out, dt) == 0);
    EXPECT(oracle_unpermute_combine(y, dt, R, H, row_of, NULL, bias, T, K, out, dt) == 0);
    void *out32 = xalloc((size_t)(T * H * 4));
    EXPECT(oracle_unpermute_combine(y, dt, R, H, row_of, w, NULL, T, K, out32, 0) == 0);
    if (gs > 0) {
        for (int p_dt = 0; p_dt < 2; ++p_dt) {
            void *part = xalloc((size_t)(n * H * (p_dt == 0 ? 4 : 2)));
            EXPECT(oracle_group_precombine(y, dt, R, H, row_of, w, idx, T, K, E, gs, slot_of, n, part, p_dt) == 0);
            EXPECT(oracle_unpermute_combine(part, p_dt, n, H, slot_of, NULL, NULL, T, G, out, dt) == 0);
            free(part);
        }
    }

    void *dout = xalloc((size_t)(T * H * esz));
    fill_rows(dout, dt, T * H);
    void *dy = xalloc((size_t)(R * H * esz));
    float *dw = xalloc(4 * (size_t)(T * K));
    EXPECT(oracle_combine_backward(dout, dt, y, dt, R, H, row_of, w, T, K, dy, dt, dw) == 0);
    void *dy2 = xalloc((size_t)(R * H * (dt == 0 ? 2 : 4)));  /* the other element type */
    EXPECT(oracle_combine_backward(dout, dt, y, dt, R, H, row_of, NULL, T, K, dy2, 1 - dt, NULL) == 0);
    free(dy2);
    float *dlog = xalloc(4 * (size_t)(T * E));
    EXPECT(oracle_route_topk_backward(idx, w, dw, T, E, K, dlog) == 0);

    for (int32_t block = 1; block <= H; block *= 2) {
        if (H % block)
            continue;
        uint8_t *q = xalloc((size_t)(T * H));
        float *sc = xalloc(4 * (size_t)(T * (H / block)));
        EXPECT(oracle_quantize_fp8(x, dt, T, H, block, q, sc) == 0);
        free(q);
        free(sc);
    }

    free(logits); free(idx); free(w); free(counts); free(gl); free(kept); free(si); free(row_of); free(pp);
    free(slot_of); free(gsrc); free(esrc); free(gcnt); free(nsl); free(ssrc);
    free(x); free(xp); free(y); free(bias); free(out); free(out32); free(dout); free(dy); free(dw); free(dlog);
}

int main(void)
{
    /* argument errors: refused before any access */
    int32_t dummy = 0;
    EXPECT(oracle_route_topk(NULL, 4, 8, 2, &dummy, NULL) != 0);
    EXPECT(oracle_route_topk(NULL, 0, 8, 9, NULL, NULL) != 0); /* K > E */
    EXPECT(oracle_build_index(NULL, NULL, 4, 2, 8, 0, 0, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                              NULL, NULL, NULL) != 0);
    EXPECT(oracle_build_index(&dummy, NULL, 1, 1, 4, 2, 2, 0, &dummy, &dummy, NULL, &dummy, &dummy, NULL, NULL, NULL,
                              NULL, NULL, NULL, NULL) != 0); /* capacity with groups */
    EXPECT(oracle_permute(NULL, 4, 8, 3, &dummy, 1, &dummy) != 0);
    EXPECT(oracle_capacity(-1, 2, 8, 5, 4) < 0);
    EXPECT(oracle_capacity(1024, 2, 8, 5, 4) == 320);

    /* shapes: T, E, K, H, dtype, capacity, group size, alignment, holes, repeated experts, limited */
    const int64_t Ts[] = {0, 1, 7, 64, 300};
    for (size_t ti = 0; ti < sizeof Ts / sizeof Ts[0]; ++ti) {
        const int64_t T = Ts[ti];
        for (int dt = 0; dt < 2; ++dt) {
            one_case(T, 8, 2, 16, dt, 0, 0, 0, 0, 0, 0);
            one_case(T, 8, 2, 16, dt, 0, 0, 0, 1, 1, 0);
            one_case(T, 12, 5, 24, dt, 3, 0, 0, 1, 0, 0);
            one_case(T, 16, 4, 8, dt, 1, 0, 0, 0, 1, 0);
            one_case(T, 16, 8, 40, dt, 0, 4, 0, 1, 0, 0);
            one_case(T, 16, 8, 40, dt, 0, 4, 0, 0, 0, 1);
            one_case(T, 9, 3, 5, dt, 0, 3, 0, 1, 1, 1);
            one_case(T, 16, 4, 32, dt, 0, 0, 8, 1, 0, 0);
            one_case(T, 16, 4, 32, dt, 0, 2, 4, 1, 1, 0);
            one_case(T, 1, 1, 1, dt, 0, 0, 0, 0, 0, 0);
            one_case(T, 32, 32, 64, dt, 0, 1, 0, 1, 0, 0);
        }
    }
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer driver: all calls clean\n");
    return 0;
}
