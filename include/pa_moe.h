/*
 * pa_moe.h — MoE routing path for MI355X (gfx950), C ABI.
 *
 * The steps around the expert GEMMs of a mixture-of-experts layer, as the
 * source pages lay them out:
 *   [cd0d9e1a]  project_6 commit cd0d9e1a, qwen3_6_scripts — the MoE prefill
 *               rewrite (256 experts, top_k = 8): flatten the T x K
 *               token-expert assignments, sort them by expert id so each
 *               expert's rows are contiguous, run the experts on contiguous
 *               rows, and add the weighted expert outputs back to their tokens
 *               in one scatter (index_add_).
 *   [490ff98a]  project_6 commit 490ff98a, Dockerfile — the router's
 *               topk_softmax kernel.
 * The expert GEMMs and their activation (between permute and combine) need
 * trained weights and are not part of this library.
 *
 * Conventions shared by every entry point:
 *   - every array is a device pointer owned by the caller (row-major,
 *     contiguous, 16-byte aligned for the hidden-row arrays, 4-byte for the
 *     rest); the library never allocates, frees or synchronises;
 *   - calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and hold no state;
 *   - invalid sizes or pointers return a negative status (the PA_* codes of
 *     pa_decode.h) before anything is launched; T == 0 is a no-op;
 *   - results are bitwise reproducible: integer results are exact, the
 *     combine sums in the fixed order j = 0 .. K-1 in fp32;
 *   - data errors (ids, pair indices or positions outside their ranges) give
 *     undefined results, never out-of-bounds accesses: such values are
 *     clamped into range.
 * Pair index a = t * K + j names the j-th choice of token t.
 */
#ifndef PA_MOE_H
#define PA_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_MOE_MAX_EXPERTS 1024
#define PA_MOE_MAX_TOPK 32

/* Router ([490ff98a] topk_softmax): p = softmax(logits[t, :]) over the E
 * experts in fp32; the K experts with the largest logits, in descending
 * order, a tie going to the lower expert id (the comparison is on the fp32
 * logits themselves, so it is exact). topk_weights[t, j] = p of the j-th
 * choice, divided by the sum of the K chosen p when renormalize != 0.
 *   logits        float32 [T, E]     (1 <= E <= 1024)
 *   topk_weights  float32 [T, K]     (1 <= K <= min(E, 32))
 *   topk_ids      int32   [T, K]                                        */
int pa_moe_topk_softmax(float* topk_weights, int32_t* topk_ids, const float* logits, int32_t T, int32_t E,
                        int32_t K, int renormalize, void* stream);

/* Bytes of device workspace pa_moe_sort_by_expert needs for these sizes
 * (or a negative status). */
int64_t pa_moe_sort_workspace_bytes(int32_t T, int32_t E, int32_t K);

/* Sort the T*K pairs by expert id ([cd0d9e1a] MoE rewrite, steps 1-2), stably
 * (ascending pair index within an expert):
 *   sorted_pairs    int32 [T*K]   pair index at each sorted position
 *   pair_pos        int32 [T*K]   sorted position of each pair (the inverse)
 *   expert_offsets  int32 [E+1]   expert e's rows are [offsets[e], offsets[e+1])
 *   topk_ids        int32 [T, K]  values in [0, E)
 *   workspace       >= pa_moe_sort_workspace_bytes(T, E, K) bytes, 4-byte
 *                   aligned; its contents on entry do not matter.
 * Four launches (per-chunk ranks and counts, a scan over chunks per expert,
 * the expert offsets, the scatter), or one single-workgroup launch for up to
 * 4096 pairs; both give the same result. */
int pa_moe_sort_by_expert(int32_t* sorted_pairs, int32_t* pair_pos, int32_t* expert_offsets,
                          const int32_t* topk_ids, int32_t T, int32_t E, int32_t K, void* workspace,
                          int64_t workspace_bytes, void* stream);

/* Lay the expert inputs out in sorted order ([cd0d9e1a] MoE rewrite, step 3:
 * contiguous rows per expert): x_sorted[pair_pos[t*K + j], :] = x[t, :] for
 * every token t and choice j; with pair_pos from pa_moe_sort_by_expert this is
 * x_sorted[i, :] = x[sorted_pairs[i] / K, :]. Done token-major: each row of x
 * is read once and written to its K positions.
 *   x         [T, hidden]     dtype (pa_dtype of pa_decode.h: f32, bf16, f16)
 *   pair_pos  int32 [T*K]     a permutation of 0..T*K-1 (if it is not, rows
 *                             that two pairs name get either one's row and
 *                             rows no pair names are left as they were)
 *   x_sorted  [T*K, hidden]   dtype; hidden * element size must be a
 *                             multiple of 16 bytes                        */
int pa_moe_permute(void* x_sorted, const void* x, const int32_t* pair_pos, int32_t T, int32_t K, int32_t hidden,
                   int32_t dtype, void* stream);

/* Weighted scatter-back of the expert outputs ([cd0d9e1a] MoE rewrite, step
 * 5, the index_add_): out[t, :] = sum_{j<K} topk_weights[t, j] *
 * y_sorted[pair_pos[t*K + j], :], accumulated in fp32 in the order
 * j = 0..K-1 and rounded once to dtype. Written as a gather per token (no
 * atomics), so every output row is written exactly once.
 *   y_sorted  [T*K, hidden]  dtype;  out [T, hidden] dtype               */
int pa_moe_combine(void* out, const void* y_sorted, const float* topk_weights, const int32_t* pair_pos,
                   int32_t T, int32_t K, int32_t hidden, int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MOE_H */
