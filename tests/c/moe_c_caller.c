/*
 * A plain C11 caller of libmoe_dispatch.so: no Python, no torch, only the HIP runtime for device
 * memory. It shows that the boundary in include/moe_dispatch.h is usable from C as it stands.
 *
 *   moe_c_caller check
 *       calls that launch nothing: status strings, capacity, row count, workspace size, and
 *       argument errors reported before any launch; prints "ok" (no GPU needed).
 *   moe_c_caller run IN OUT
 *       IN:  int64 T, E, K, H; float32 logits[T*E]; bf16 bits x[T*H]; bf16 bits y[T*K*H]
 *       runs route -> index -> source-major permute -> combine on the GPU (standard mode) and
 *       writes OUT: int32 topk_idx[T*K]; float32 topk_w[T*K]; int32 counts[E],
 *       group_list[E], sorted_indices[R], row_of[T*K]; float32 permuted_probs[R];
 *       bf16 bits xp[R*H] (permuted x), out[T*H] (combined y), with R = T*K.
 * Exit status 0 on success; 2 HIP error, 3 library error, 4 I/O or usage error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_dispatch.h"

#define CHECK_HIP(x)                                                                   \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));             \
            return 2;                                                                  \
        }                                                                              \
    } while (0)

#define CHECK_MOE(x)                                                                   \
    do {                                                                               \
        moe_status s_ = (x);                                                           \
        if (s_ != MOE_OK) {                                                            \
            fprintf(stderr, "%s failed: %s\n", #x, moe_status_string(s_));             \
            return 3;                                                                  \
        }                                                                              \
    } while (0)

#define EXPECT(c)                                                                      \
    do {                                                                               \
        if (!(c)) {                                                                    \
            fprintf(stderr, "check failed: %s\n", #c);                                 \
            return 3;                                                                  \
        }                                                                              \
    } while (0)

static int check_host_calls(void)
{
    size_t ws = 0;
    int dummy = 0;
    void *fake = &dummy; /* never dereferenced: validation fails before any launch */
    EXPECT(moe_status_string(MOE_OK) != NULL && moe_status_string(MOE_ERR_INVALID) != NULL);
    EXPECT(moe_expert_capacity(8192, 8, 128, 5, 4) == 640);
    EXPECT(moe_expert_capacity(-1, 8, 128, 5, 4) == -1);
    EXPECT(moe_index_rows(16384, 8, 256, 0, 0) == 16384 * 8);
    EXPECT(moe_index_rows(16384, 8, 256, 0, 128) == 16384 * 8 + 256 * 127);
    EXPECT(moe_index_rows(8192, 8, 128, 640, 0) == 128 * 640);
    EXPECT(moe_build_index_workspace_size(16384, 8, 256, 0, &ws) == MOE_OK && ws > 0);
    EXPECT(moe_route_topk((const float *)fake, 4, 8, 9, (int32_t *)fake, (float *)fake, NULL) == MOE_ERR_INVALID);
    EXPECT(moe_route_topk((const float *)fake, 4, 2048, 2, (int32_t *)fake, (float *)fake, NULL) ==
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_route_topk(NULL, 0, 8, 2, NULL, NULL, NULL) == MOE_OK); /* empty: nothing launched */
    EXPECT(moe_unpermute_combine(fake, MOE_FP8_E4M3, 1, 8, (const int32_t *)fake, NULL, NULL, 1, 1, fake, MOE_BF16,
                                 NULL) == MOE_ERR_UNSUPPORTED);
    printf("ok\n");
    return 0;
}

static int read_all(FILE *f, void *p, size_t bytes)
{
    return fread(p, 1, bytes, f) == bytes ? 0 : 4;
}

static int run(const char *in_path, const char *out_path)
{
    FILE *f = fopen(in_path, "rb");
    if (!f)
        return 4;
    int64_t hdr[4];
    if (read_all(f, hdr, sizeof hdr)) {
        fclose(f);
        return 4;
    }
    const int64_t T = hdr[0], E = hdr[1], K = hdr[2], H = hdr[3];
    if (T < 1 || E < 1 || K < 1 || K > E || H < 1 || T * K > (1 << 24) || H > (1 << 16)) {
        fclose(f);
        return 4;
    }
    const int64_t R = moe_index_rows(T, (int32_t)K, (int32_t)E, 0, 0);
    EXPECT(R == T * K);
    const size_t n_logits = (size_t)(T * E), n_x = (size_t)(T * H), n_y = (size_t)(R * H), n_tk = (size_t)(T * K);
    float *h_logits = malloc(n_logits * sizeof(float));
    uint16_t *h_x = malloc(n_x * 2), *h_y = malloc(n_y * 2);
    if (!h_logits || !h_x || !h_y || read_all(f, h_logits, n_logits * 4) || read_all(f, h_x, n_x * 2) ||
        read_all(f, h_y, n_y * 2)) {
        fclose(f);
        return 4;
    }
    fclose(f);

    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    float *d_logits, *d_w, *d_probs;
    int32_t *d_idx, *d_counts, *d_gl, *d_sorted, *d_row_of;
    uint16_t *d_x, *d_y, *d_xp, *d_out;
    void *d_ws = NULL;
    size_t ws = 0;
    CHECK_MOE(moe_build_index_workspace_size(T, (int32_t)K, (int32_t)E, 0, &ws));
    CHECK_HIP(hipMalloc((void **)&d_logits, n_logits * 4));
    CHECK_HIP(hipMalloc((void **)&d_w, n_tk * 4));
    CHECK_HIP(hipMalloc((void **)&d_idx, n_tk * 4));
    CHECK_HIP(hipMalloc((void **)&d_counts, (size_t)E * 4));
    CHECK_HIP(hipMalloc((void **)&d_gl, (size_t)E * 4));
    CHECK_HIP(hipMalloc((void **)&d_sorted, (size_t)R * 4));
    CHECK_HIP(hipMalloc((void **)&d_row_of, n_tk * 4));
    CHECK_HIP(hipMalloc((void **)&d_probs, (size_t)R * 4));
    CHECK_HIP(hipMalloc((void **)&d_x, n_x * 2));
    CHECK_HIP(hipMalloc((void **)&d_y, n_y * 2));
    CHECK_HIP(hipMalloc((void **)&d_xp, n_y * 2));
    CHECK_HIP(hipMalloc((void **)&d_out, n_x * 2));
    if (ws > 0)
        CHECK_HIP(hipMalloc(&d_ws, ws));
    CHECK_HIP(hipMemcpy(d_logits, h_logits, n_logits * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_x, h_x, n_x * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_y, h_y, n_y * 2, hipMemcpyHostToDevice));

    moe_index ix;
    memset(&ix, 0, sizeof ix);
    ix.counts = d_counts;
    ix.group_list = d_gl;
    ix.sorted_indices = d_sorted;
    ix.row_of = d_row_of;
    ix.permuted_probs = d_probs;
    CHECK_MOE(moe_route_topk(d_logits, T, (int32_t)E, (int32_t)K, d_idx, d_w, s));
    CHECK_MOE(moe_build_index(d_idx, d_w, T, (int32_t)K, (int32_t)E, 0, 0, 0, &ix, d_ws, ws, s));
    CHECK_MOE(moe_permute_scatter(d_x, T, H, MOE_BF16, d_row_of, (int32_t)K, d_sorted, R, d_xp, s));
    CHECK_MOE(moe_unpermute_combine(d_y, MOE_BF16, R, H, d_row_of, d_w, NULL, T, (int32_t)K, d_out, MOE_BF16, s));
    CHECK_HIP(hipStreamSynchronize(s));

    FILE *o = fopen(out_path, "wb");
    if (!o)
        return 4;
    struct {
        const void *dev;
        size_t bytes;
    } parts[] = {{d_idx, n_tk * 4},      {d_w, n_tk * 4},         {d_counts, (size_t)E * 4},
                 {d_gl, (size_t)E * 4},  {d_sorted, (size_t)R * 4}, {d_row_of, n_tk * 4},
                 {d_probs, (size_t)R * 4}, {d_xp, n_y * 2},        {d_out, n_x * 2}};
    for (size_t i = 0; i < sizeof parts / sizeof parts[0]; ++i) {
        void *h = malloc(parts[i].bytes);
        if (!h) {
            fclose(o);
            return 4;
        }
        CHECK_HIP(hipMemcpy(h, parts[i].dev, parts[i].bytes, hipMemcpyDeviceToHost));
        if (fwrite(h, 1, parts[i].bytes, o) != parts[i].bytes) {
            free(h);
            fclose(o);
            return 4;
        }
        free(h);
    }
    fclose(o);
    hipFree(d_logits);
    hipFree(d_w);
    hipFree(d_idx);
    hipFree(d_counts);
    hipFree(d_gl);
    hipFree(d_sorted);
    hipFree(d_row_of);
    hipFree(d_probs);
    hipFree(d_x);
    hipFree(d_y);
    hipFree(d_xp);
    hipFree(d_out);
    if (d_ws)
        hipFree(d_ws);
    CHECK_HIP(hipStreamDestroy(s));
    free(h_logits);
    free(h_x);
    free(h_y);
    printf("ok T=%lld E=%lld K=%lld H=%lld\n", (long long)T, (long long)E, (long long)K, (long long)H);
    return 0;
}

int main(int argc, char **argv)
{
    if (argc == 2 && strcmp(argv[1], "check") == 0)
        return check_host_calls();
    if (argc == 4 && strcmp(argv[1], "run") == 0)
        return run(argv[2], argv[3]);
    fprintf(stderr, "usage: %s check | run IN OUT\n", argv[0]);
    return 4;
}
