/*
 * moe_dispatch.h -- C ABI of the MI355X (gfx950) MoE token dispatch / unpermute-combine library
 * (libmoe_dispatch.so).
 *
 * The operations follow these web pages (cited by title and section):
 *   [Combine]   "03 · Combine 与 forward / backward 对称性" (llm-infra-atlas, EP chapter)
 *   [Scratch]   "从零理解 MoE 算子：路由、专家并行与 Token 重排" (171host)
 *   [CANN]      CANN Dispatch&Combine optimisation notes (cann.csdn.net), "Dispatch&Combine优化"
 *   [Megatron]  "token dispatcher + fuse_a2a" (obnotes, Megatron/transformer-moe)
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE memory owned by the caller (the library never allocates
 *     and never frees). Tensors are row-major and contiguous. Indices and counts are int32,
 *     router weights and probabilities float32, hidden rows float32 or bf16 (moe_dtype).
 *   - Calls are asynchronous: they enqueue kernels on `stream` (a hipStream_t; NULL is the
 *     null stream) and return. Results are visible to later work on the same stream.
 *   - Argument errors are reported synchronously, before anything is launched:
 *     MOE_ERR_INVALID (null pointer where data is needed, negative size, K < 1, K > E,
 *     H < 1, group size not dividing E, ...) or MOE_ERR_UNSUPPORTED (E > 1024, K > 32, a
 *     hidden row longer than 2^31 - 1 bytes, more than 2^31 - 1 tokens, or a combination the
 *     call does not implement). MOE_ERR_HIP means a launch failed.
 *   - A size of zero tokens / rows is valid (an empty rank or an expert with no tokens must
 *     work, [Scratch] §26.1-26.2): a call with nothing to write launches nothing, and
 *     moe_build_index with T = 0 still writes its per-expert results (zero counts) and the
 *     marks of its rows (padding or unused).
 *   - Memory safety does not depend on the data: an expert id outside [0, E) routes nowhere
 *     (the pages write -1 for "no expert"), a row index outside the source range selects a
 *     zero row (permute) or no term (combine). Expert ids in one row of topk_idx must be
 *     distinct for the pages' routing map to be defined; if they repeat, slots of the same
 *     expert are ordered by slot.
 *   - The library holds no global state (apart from the scratch of moe_build_index_noalloc);
 *     calls on different streams may run concurrently as long as they do not write the same
 *     memory.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_HIP = 3
} moe_status;

/* Element types of hidden rows. MOE_FP8_E4M3 (1-byte OCP E4M3 codes, the FP8 dispatch) is
 * accepted by the permutes only, which copy bytes; the combines work in bf16 / float32 and
 * return MOE_ERR_UNSUPPORTED for it. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Upper limits of the kernels. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/* Markers in gather maps (sorted_indices, esrc): a padding row, written as zeros by the
 * permutes; and an unused row after the last expert segment (buffer slack when the buffer is
 * sized by an upper bound), which no call writes. */
#define MOE_ROW_PAD (-1)
#define MOE_ROW_UNUSED (-2)

/* Static, human-readable name of a status code. Never NULL. */
const char *moe_status_string(moe_status s);

/* Expert capacity, [Scratch] §18: ceil(tokens * top_k / num_experts * capacity_factor) with the
 * capacity factor given as the exact fraction cf_num / cf_den (1.25 = 5/4), computed in
 * integers on the host. 1024 tokens, top_k 2, 8 experts, 5/4 -> 320.
 * Returns -1 for tokens < 0, top_k < 1, num_experts < 1, cf_num < 0, cf_den < 1 or a result
 * that does not fit in int32. */
int64_t moe_expert_capacity(int64_t tokens, int32_t top_k, int32_t num_experts,
                            int32_t cf_num, int32_t cf_den);

/* Top-k routing, [Scratch] §3 and §27: for each token t the K experts with the largest logits,
 * then a softmax over those K logits only.
 *   logits   [T, E] float32, finite.
 *   topk_idx [T, K] int32 out: slot k is the k-th expert in the order (logit descending,
 *            expert id ascending); equal logits (+0 and -0 are equal) go to the lower id.
 *   topk_w   [T, K] float32 out: w_k = exp(s_k - s_0) / sum_j exp(s_j - s_0), evaluated in
 *            double (the router softmax is precision sensitive, [Scratch] §26.7) and rounded
 *            once to float32; the sum runs in slot order.
 * Requires 1 <= K <= E, E <= MOE_MAX_EXPERTS, K <= MOE_MAX_TOPK. */
moe_status moe_route_topk(const float *logits, int64_t T, int32_t E, int32_t K,
                          int32_t *topk_idx, float *topk_w, hipStream_t stream);

/* Group-limited routing, [Scratch] §21: the experts form G = E / group_size contiguous groups
 * (g = e / group_size; a group stands for a rank or node); the router first keeps the
 * topk_groups groups with the best scores, then picks the top K experts among the experts of
 * those groups only, and the weights are the softmax over the K selected logits exactly as in
 * moe_route_topk. A group's score is its largest logit (the pages define no score: with the
 * maximum, topk_groups = G is plain routing and the token's best expert is always kept); equal
 * scores go to the lower group id. A token's K experts then lie in at most topk_groups groups,
 * so the group dispatch sends each token at most topk_groups times.
 * Requires group_size dividing E, 1 <= topk_groups <= G, K <= topk_groups * group_size
 * (else MOE_ERR_INVALID) and G <= 256 (else MOE_ERR_UNSUPPORTED). */
moe_status moe_route_topk_grouped(const float *logits, int64_t T, int32_t E, int32_t K, int32_t group_size,
                                  int32_t topk_groups, int32_t *topk_idx, float *topk_w, hipStream_t stream);

/* The dispatch "handle" ([Combine] §3: computed once by dispatch, reused by combine).
 * All members are caller-owned device arrays, written by moe_build_index.
 * R = moe_index_rows(...): T*K in the standard and group modes, E*capacity in drop-and-pad
 * mode, T*K + E*(alignment-1) with expert alignment. */
typedef struct moe_index {
    int32_t *counts;         /* [E] rows routed to each expert, before capacity ([Megatron] §1.2
                                num_tokens_per_expert). Required. */
    int32_t *group_list;     /* [E] inclusive running sum of counts ([Scratch] §7:
                                [3,2,4] -> [3,5,9]); in the standard and group modes expert e
                                owns rows [group_list[e]-counts[e], group_list[e]). With expert
                                alignment A the running sum of the aligned lengths
                                ceil(counts/A)*A (expert e's segment ends at group_list[e], its
                                tokens come first, then padding rows). In drop-and-pad mode it
                                stays the running sum of the counts before capacity and
                                describes no row layout: there expert e owns rows
                                [e*capacity, e*capacity + kept_counts[e]), then padding up to
                                (e+1)*capacity. Required. */
    int32_t *kept_counts;    /* [E] min(counts, capacity) in drop-and-pad mode, counts
                                otherwise. May be NULL. */
    int32_t *sorted_indices; /* [R] source token of each expert-major row ([Megatron] §1.1,
                                masked_select over the transposed routing map): experts in
                                ascending order, tokens ascending inside an expert. Padding
                                rows hold MOE_ROW_PAD (-1), rows after the last segment
                                MOE_ROW_UNUSED (-2). Required. */
    int32_t *row_of;         /* [T, K] expert-major row of slot (t,k), -1 if the slot routes
                                nowhere or was dropped (the saved mapping that makes the permute
                                invertible, [Scratch] §26.5). Required. */
    float *permuted_probs;   /* [R] topk_w of the slot in each row ([Megatron] §1.1 step 4),
                                0 on padding/unused rows, 1 if topk_w is NULL. May be NULL. */
    /* group mode only (group_size > 0), else ignored; all required in group mode: */
    int32_t *slot_of;        /* [T, G] slot of (token t, group g) in the send-once list, -1 if
                                token t uses no expert of group g ([CANN] §1(1)). */
    int32_t *gsrc;           /* [T*min(K,G)] source token of each group slot, groups ascending
                                then tokens ascending; only the first n_slots entries are
                                written. */
    int32_t *esrc;           /* [R] group slot feeding each expert-major row; MOE_ROW_PAD on
                                padding rows, MOE_ROW_UNUSED after the last segment. */
    int32_t *group_counts;   /* [G] slots per group. */
    int32_t *n_slots;        /* [1] number of group slots M_g (the caller reads it back if it
                                needs the exact size; gsrc may be sized by the upper bound). */
    int32_t *slot_src;       /* [T, K] group mode, may be NULL (not written): the group slot
                                feeding routing slot (t,k), i.e. slot_of[t, group of its expert]
                                = esrc[row_of[t,k]]; -1 if the slot routes nowhere. The receive
                                side passes it to moe_permute_grouped as src_of, so that each
                                destination's source is known without a lookup. */
} moe_index;

/* Rows R of the expert-major arrays (sorted_indices, permuted_probs, esrc) and buffers for
 * these sizes: E*capacity with capacity > 0, else T*K + E*(alignment-1) (alignment <= 1: T*K),
 * the most that the segments rounded up to a multiple of the alignment can need. Returns -1 for
 * invalid sizes, capacity together with alignment > 1, or R above 2^31 - 1. */
int64_t moe_index_rows(int64_t T, int32_t K, int32_t E, int32_t capacity, int32_t alignment);

/* Bytes of device workspace that moe_build_index needs for these sizes: the tile counts of the
 * experts (and of the groups), at most 128 tiles. The caller allocates it, 16-byte aligned
 * (NULL when the size is 0); its contents need no initialisation and mean nothing after the
 * call. */
moe_status moe_build_index_workspace_size(int64_t T, int32_t K, int32_t E, int32_t group_size,
                                          size_t *bytes);

/* Builds the expert-major index from the routing result ([Megatron] §1.1; [Scratch] §6, §7,
 * §11-13, §16).
 *   topk_idx [T, K] int32 expert ids (-1 or any id outside [0, E) = no expert).
 *   topk_w   [T, K] float32 or NULL (then permuted_probs holds 1 on routed rows).
 *   capacity > 0 selects drop-and-pad ([Scratch] §18, §26.6): expert e owns rows
 *            [e*capacity, (e+1)*capacity); the p-th token of expert e (tokens in ascending
 *            order) is kept at row e*capacity + p iff p < capacity, later ones are dropped
 *            (row_of = -1) and the rest of the expert's rows are padding.
 *   group_size > 0 selects group mode ([CANN] §1(1)): experts e form G = E / group_size
 *            contiguous groups g = e / group_size, and slot_of/gsrc/esrc/group_counts/n_slots
 *            are written. capacity > 0 together with group_size > 0 is MOE_ERR_UNSUPPORTED.
 *   alignment > 1 selects expert alignment ([Combine] §6, dispatch(..., expert_alignment=128)):
 *            each expert segment is rounded up to a multiple of the alignment, its tokens first
 *            and MOE_ROW_PAD rows after them, so that every segment of the grouped GEMM input
 *            starts at a multiple of the alignment; group_list follows the aligned segments.
 *            Not with capacity (MOE_ERR_UNSUPPORTED); 0 or 1 means none.
 * Rows after the last segment are MOE_ROW_UNUSED. The build is deterministic: no position
 * depends on the timing of atomics. */
moe_status moe_build_index(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K,
                           int32_t E, int32_t capacity, int32_t group_size, int32_t alignment,
                           const moe_index *out, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* moe_build_index without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * tile counts go to a scratch array inside the library instead -- 1 MiB of device memory per GPU,
 * enough for every input moe_build_index accepts (at most 128 tiles of 1024 expert and 1024 group
 * counts), held by each GPU the library runs on until the process ends. Nothing is allocated;
 * arguments, results and errors are those of moe_build_index (bit for bit the same arrays), plus:
 *   - the stream must belong to the current device (else MOE_ERR_INVALID): the scratch used is
 *     the current device's, whose address is looked up on the first call on that device
 *     (MOE_ERR_HIP if that fails);
 *   - a plan larger than the scratch returns MOE_ERR_UNSUPPORTED (no valid input makes one);
 *   - every call on one GPU shares that GPU's scratch: calls on the same stream are ordered, but
 *     calls that overlap on one GPU (different streams, or different host threads without
 *     ordering between their streams) race and may write wrong results. The scratch needs no
 *     clearing: each call writes the counts it reads. */
moe_status moe_build_index_noalloc(const int32_t *topk_idx, const float *topk_w, int64_t T, int32_t K,
                                   int32_t E, int32_t capacity, int32_t group_size, int32_t alignment,
                                   const moe_index *out, hipStream_t stream);

/* Routing and index build in one call ([Scratch] §3, §27: top-k and the softmax over the K
 * selected logits; §7: the per-expert counts behind group_list; [Megatron] §1.1: the index):
 * the same topk_idx, topk_w and moe_index arrays, bit for bit, as moe_route_topk (route_group_size
 * <= 0) or moe_route_topk_grouped(route_group_size, topk_groups) followed by moe_build_index(
 * topk_idx, topk_w, T, K, E, capacity, group_size, alignment, ...). Where moe_build_index would
 * count its tiles in a launch of its own, the workgroups that route a tile count its slots
 * instead, one launch fewer. Arguments are those of the two calls (route_group_size and
 * topk_groups as moe_route_topk_grouped's group_size and topk_groups; group_size is the index's);
 * the workspace (16-byte aligned; contents need no initialisation and mean nothing after the
 * call) must hold moe_route_topk_index_workspace_size bytes. Every argument error of either call
 * is returned before anything is launched. */
moe_status moe_route_topk_index_workspace_size(int64_t T, int32_t K, int32_t E, int32_t group_size, size_t *bytes);
moe_status moe_route_topk_index(const float *logits, int64_t T, int32_t E, int32_t K, int32_t route_group_size,
                                int32_t topk_groups, int32_t *topk_idx, float *topk_w, int32_t capacity,
                                int32_t group_size, int32_t alignment, const moe_index *out, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Row gather ([Megatron] §1.1 step 5, permuted_input = tokens.index_select(0, sorted_indices);
 * [Scratch] §12, permuted_tokens = tokens[permute_indices]):
 *   dst[i, :] = src[src_row[i], :] copied bit for bit, for i in [0, N); a src_row outside
 *   [0, src_rows) (MOE_ROW_PAD of padding rows) writes a row of zeros, except MOE_ROW_UNUSED,
 *   which leaves row i untouched (this holds for every call that takes a gather map).
 *   src [src_rows, H] of dtype dt, src_row [N] int32, dst [N, H] of dtype dt.
 * Used for the standard dispatch (src_row = sorted_indices, N = R), drop-and-pad (which also
 * zero-fills the padding rows) and the two stages of the group dispatch (src_row = gsrc, then
 * esrc). moe_permute_scatter below computes the same rows reading each source row once. */
moe_status moe_permute(const void *src, int64_t src_rows, int64_t H, moe_dtype dt,
                       const int32_t *src_row, int64_t N, void *dst, hipStream_t stream);

/* The same row copy as moe_permute, taken source-major: each source row is read once and
 * written to every destination that names it, instead of being read again for each destination
 * (with top-k routing a token row feeds K expert rows, [Scratch] §4).
 *   dst_of  [src_rows, J] int32: dst[dst_of[t*J + j], :] = src[t, :] for every entry in [0, N);
 *           other entries (-1) are skipped. J <= MOE_MAX_EXPERTS (one column per expert group
 *           at most); the entries are read 64 at a time, so a wide map costs a little more.
 *   src_row [N] int32 or NULL: rows i with src_row[i] outside [0, src_rows) are written as zeros
 *           (the padding rows of drop-and-pad); NULL writes no zero rows.
 * When dst_of is the inverse of src_row -- row_of and sorted_indices of one moe_index are -- the
 * result is bit for bit that of moe_permute(src, src_rows, H, dt, src_row, N, dst). Every
 * destination row must be named at most once; rows named by neither map are left untouched. */
moe_status moe_permute_scatter(const void *src, int64_t src_rows, int64_t H, moe_dtype dt,
                               const int32_t *dst_of, int32_t J, const int32_t *src_row, int64_t N,
                               void *dst, hipStream_t stream);

/* The row gather of moe_permute, worked through in groups of destination rows: the result is
 * defined by the gather map alone,
 *   dst[r, :] = src[src_row[r], :]   (bit for bit) for every r listed in dst_of,
 *   dst[r, :] = 0                     for every r in [0, N) with src_row[r] outside [0, src_rows),
 * and dst_of only decides which rows are copied together: within one group (a row of dst_of),
 * a source row named by several destinations is read once. This is the receive side of the
 * send-once-per-rank dispatch ([CANN] §1(1)) put back in expert-major order ([Scratch] §11-12,
 * rank-major to expert-major): src = the group buffer, src_row = moe_index.esrc, dst_of =
 * moe_index.row_of (one group per token, J = K), where each group slot feeds every expert of
 * its group that the token chose.
 *   src     [src_rows, H] (dt); src_row [N] int32 (required); dst [N, H] (dt).
 *   dst_of  [M, J] int32 destination rows, J <= 64; entries outside [0, N) are ignored. A row
 *           may be listed more than once (each copy writes the same bytes); rows with a valid
 *           src_row that dst_of never lists are left untouched.
 *   src_of  [M, J] int32 or NULL: the source row of each listed destination, which must equal
 *           src_row[dst_of[m*J + j]] (moe_index.slot_src is that for the group receive); with it
 *           the sources load together with the destinations instead of after them. Its entries
 *           for unlisted columns (dst_of outside [0, N)) are ignored. The result is the same.
 * With dst_of = the inverse of src_row (every row listed), the result equals
 * moe_permute(src, src_rows, H, dt, src_row, N, dst) bit for bit. */
moe_status moe_permute_grouped(const void *src, int64_t src_rows, int64_t H, moe_dtype dt,
                               const int32_t *src_row, int64_t N, const int32_t *dst_of, int64_t M,
                               int32_t J, const int32_t *src_of, void *dst, hipStream_t stream);

/* FP8 dispatch ([Combine] §3: the dispatch sends FP8, the combine stays BF16; the DeepEP
 * dispatch call in [Megatron] passes x together with x_scales, num_scales scale groups per token
 * along the hidden dimension). Each token's row is cut into H / block blocks of `block`
 * consecutive elements; per block
 *   amax = max |x|,  scale = amax / 448 (float32 division; 1 when amax is 0),
 *   q[i] = E4M3 code of x[i] / scale (float32 division, nearest even, saturating at 448),
 * E4M3 being the OCP 8-bit format (bias 7, no infinities, 448 the largest finite value).
 * x must be finite (then |x / scale| exceeds 448 by at most the division's rounding and the
 * code is at most 448 in magnitude).
 *   moe_quantize_fp8: x [T, H] (x_dt float32 or bf16) -> q [T, H] bytes, scales [T, H/block]
 *     float32. block must divide H.
 *   moe_permute_scatter_fp8: the same codes and scales, computed once per source row and
 *     written source-major like moe_permute_scatter: dst[dst_of[t*J+j]] = q[t],
 *     dst_scales[...] = scales[t]; rows with src_row outside [0, src_rows) get zero codes and
 *     zero scales (padding), MOE_ROW_UNUSED rows are left untouched. Equal, bit for bit, to
 *     moe_quantize_fp8 followed by moe_permute_scatter of the codes (MOE_FP8_E4M3) and of the
 *     scales (float32, H / block columns). block must be a power of two in [8, 1024] dividing H
 *     (else MOE_ERR_UNSUPPORTED), J <= MOE_MAX_EXPERTS, src and dst 16-byte aligned.
 * The moved rows then hold half the bytes of bf16 rows; moe_permute / moe_permute_grouped move
 * FP8 rows (and float32 scale rows) as they move any rows. */
moe_status moe_quantize_fp8(const void *x, moe_dtype x_dt, int64_t T, int64_t H, int32_t block, uint8_t *q,
                            float *scales, hipStream_t stream);
moe_status moe_permute_scatter_fp8(const void *src, moe_dtype src_dt, int64_t src_rows, int64_t H, int32_t block,
                                   const int32_t *dst_of, int32_t J, const int32_t *src_row, int64_t N, uint8_t *dst,
                                   float *dst_scales, hipStream_t stream);

/* The receive side of the FP8 group dispatch: FP8 rows and their scale rows moved together, in one
 * launch ([Combine] §3 and the DeepEP dispatch call in [Megatron]: the codes travel with their
 * scales; [CANN] §1(1), [Scratch] §11-12: group slots back to expert-major rows). Bit for bit
 * moe_permute_grouped of the codes (MOE_FP8_E4M3 rows of H bytes) followed by moe_permute_grouped
 * of the scales (float32 rows of H / block values) with the same src_row, dst_of and src_of:
 * every listed row gets its source's codes and scales, every row whose src_row lies outside
 * [0, src_rows) (MOE_ROW_UNUSED excepted) gets zero codes and zero scales.
 *   src [src_rows, H] codes, src_scales [src_rows, H/block] float32, dst [N, H], dst_scales
 *   [N, H/block]; block >= 1 must divide H (else MOE_ERR_INVALID); the other arguments, limits
 *   and errors as in moe_permute_grouped. The group dispatch's receive:
 *   moe_permute_grouped_fp8(codes, scales, ..., moe_index.esrc, R, moe_index.row_of, T, K,
 *   moe_index.slot_src, ...) after moe_permute_scatter_fp8 over moe_index.slot_of. */
moe_status moe_permute_grouped_fp8(const uint8_t *src, const float *src_scales, int64_t src_rows, int64_t H,
                                   int32_t block, const int32_t *src_row, int64_t N, const int32_t *dst_of,
                                   int64_t M, int32_t J, const int32_t *src_of, uint8_t *dst, float *dst_scales,
                                   hipStream_t stream);

/* Unpermute + weighted top-k merge ([Combine] §1: out[t] = sum over the token's top-k experts
 * of probs[t,e] * expert_e(x[t]); [Scratch] §13, §16):
 *   out[t, :] = sum_{k = 0..K-1, row_of[t,k] in [0, y_rows)} w[t,k] * y[row_of[t,k], :]
 * with a float32 accumulator starting at +0 and one fused multiply-add per term in slot order
 * k = 0, 1, ..., K-1 (deterministic: no atomics, no reordering), then stored as float32 or
 * rounded to bf16 (nearest, ties to even).
 *   y      [y_rows, H] expert outputs in expert-major order (dtype y_dt).
 *   row_of [T, K] int32 (moe_index.row_of).
 *   w      [T, K] float32, or NULL for unit weights (the pure-add combine, [Combine] §3).
 *   bias   [T, H] of dtype out_dt, or NULL: the final bias of [Combine] §3, added in float32
 *          after the sum (one addition) before the output is rounded.
 *   out    [T, H] dtype out_dt.
 * K may be up to 1024 here: the group-mode final sum calls it with y = partials,
 * row_of = slot_of, w = NULL and K = G. */
moe_status moe_unpermute_combine(const void *y, moe_dtype y_dt, int64_t y_rows, int64_t H,
                                 const int32_t *row_of, const float *w, const void *bias, int64_t T,
                                 int32_t K, void *out, moe_dtype out_dt, hipStream_t stream);

/* Local pre-combine per group ([CANN] §1(2): the outputs of a token's experts on the same rank
 * are merged with their weights before leaving the rank; here a group of group_size experts
 * stands for a rank). For every (t, g) with s = slot_of[t*G + g] in [0, slots_cap):
 *   partials[s, :] = sum_{k: topk_idx[t,k] in group g, row_of[t,k] in [0, y_rows)}
 *                    w[t,k] * y[row_of[t,k], :]
 * float32, fused multiply-add in slot order, an empty sum being +0. With slot_of from
 * moe_build_index the partials are stored compactly ([n_slots, H], one row per (token,
 * group) that exists); a slot_of numbering every (t, g) gives the dense [T, G, H] layout.
 * Rows of partials not named by slot_of are left untouched.
 *   y [y_rows, H] (y_dt), row_of/topk_idx/w [T, K], slot_of [T, G], partials [slots_cap, H]
 *   of dtype partials_dt: MOE_F32 stores the float32 sums, MOE_BF16 rounds each once to bf16
 *   (nearest, ties to even) -- the BF16 exchange of [Combine] §3 (DeepEP's combine sends BF16),
 *   half the bytes; the final sum then reads bf16 partials. w may be NULL (unit weights). */
moe_status moe_group_precombine(const void *y, moe_dtype y_dt, int64_t y_rows, int64_t H,
                                const int32_t *row_of, const float *w, const int32_t *topk_idx,
                                int64_t T, int32_t K, int32_t E, int32_t group_size,
                                const int32_t *slot_of, int64_t slots_cap, void *partials,
                                moe_dtype partials_dt, hipStream_t stream);

/* Backward of moe_unpermute_combine ([Combine] §4: the combine is linear in the expert outputs,
 * so its backward is the transposed map -- a dispatch of the output gradient back to the expert
 * rows -- and the router gradient reaches only the selected slots):
 *   dy[row_of[t,k], :] = w[t,k] * dout[t, :]   (float32 product, stored as dy_dt)
 *   dw[t, k] = sum_h dout[t,h] * y[row_of[t,k], h]   (float32, summed in a fixed order: each
 *              thread's elements in order, a reduce-scatter butterfly over the wavefront, the
 *              wavefronts in order; 0 for a slot whose row is outside [0, y_rows))
 * and, when src_row is given, every row r of dy with src_row[r] outside [0, T) is written as
 * zeros (padding rows, which fed no output) -- except MOE_ROW_UNUSED rows. Each row of dy must be
 * named by at most one slot; other rows are left untouched.
 *   dout [T, H] (dout_dt); y [y_rows, H] (y_dt; may be NULL when dw is NULL); row_of, w [T, K]
 *   (w NULL: unit weights, dy = dout); src_row [y_rows] (moe_index.sorted_indices) or NULL;
 *   dy [y_rows, H] (dy_dt); dw [T, K] float32 or NULL (not computed).
 * The backward of the dispatch needs no call of its own ([Combine] §4.1): it is the unit-weight
 * combine of the expert-row gradient, moe_unpermute_combine(dxp, ..., row_of, NULL, NULL, ...); in
 * group mode moe_group_precombine with w = NULL followed by the final sum over groups. */
moe_status moe_unpermute_combine_backward(const void *dout, moe_dtype dout_dt, const void *y, moe_dtype y_dt,
                                          int64_t y_rows, int64_t H, const int32_t *row_of, const float *w,
                                          int64_t T, int32_t K, const int32_t *src_row, void *dy, moe_dtype dy_dt,
                                          float *dw, hipStream_t stream);

/* Backward of moe_route_topk's softmax over the K selected logits ([Scratch] §3, §27: the
 * softmax runs over the selected scores; [Combine] §6: only the selected experts carry router
 * gradient, the selection itself being piecewise constant). With w = topk_w, g = d_topk_w:
 *   d_logits[t, topk_idx[t,k]] += w[t,k] * (g[t,k] - sum_j w[t,j] g[t,j])
 * in double (the sum over j in slot order, the slots in order), rounded once to float32; every
 * other logit of the row gets 0. Slots with an id outside [0, E) give nothing.
 *   topk_idx, topk_w, d_topk_w [T, K]; d_logits [T, E] float32, every entry written. */
moe_status moe_route_topk_backward(const int32_t *topk_idx, const float *topk_w, const float *d_topk_w, int64_t T,
                                   int32_t E, int32_t K, float *d_logits, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H */
