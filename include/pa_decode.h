/*
 * pa_decode.h — paged-attention decode for MI355X (gfx950), C ABI.
 *
 * One query token per sequence attends to that sequence's context. The
 * context's keys and values live in fixed 16-token physical blocks of two
 * pools, reached through a per-sequence block table.
 *
 * Sources (the pages this library implements):
 *   [cd0d9e1a]   project_6 commit cd0d9e1a, qwen3_6_scripts — commit messages
 *                "paged_attn.py rewrite" (item 2: the V1/V2 heuristic) and
 *                "V2 implementation" (phase 1 partials, phase 2 log-sum-exp).
 *   [prefix-doc] project_6 blame of optimizations/prefix_prefill_patch.py —
 *                docstring parts on the model's attention shapes and on the
 *                partition-size constant.
 *
 * Definition computed by every entry point (for s < S, h < H, G = H / Hkv,
 * kv = h / G, L = seq_lens[s]):
 *     z_t  = scale * <q[s,h,:], K_t>            t < L
 *     out[s,h,:] = sum_t exp(z_t - max z) V_t / sum_t exp(z_t - max z)
 * with K_t = k_cache[block_tables[s][t / 16], kv, t % 16, :] (V_t alike).
 *
 * Layouts (all row-major, all contiguous):
 *     q            [S, H, D]                 dtype
 *     k_cache      [num_blocks, Hkv, 16, D]  dtype
 *     v_cache      [num_blocks, Hkv, 16, D]  dtype
 *     block_tables [S, max_blocks_per_seq]   int32
 *     seq_lens     [S]                       int32
 *     out          [S, H, D]                 dtype
 *     exp_sums     [S, H, Pmax]              float32  (V2 partials)
 *     max_logits   [S, H, Pmax]              float32
 *     tmp_out      [S, H, Pmax, D]           float32
 * with Pmax = ceil(max_blocks_per_seq * 16 / PS) (pa_max_partitions()), PS the
 * partition size of the shape (512 unless the shape opts into 256).
 *
 * Memory and ownership: every array pointer is a device pointer owned by the
 * caller, 16-byte aligned. The library never allocates, frees or
 * synchronises; `shape` is a host pointer read during the call only.
 * Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream). Calls hold no state and may run concurrently when their outputs
 * and partial buffers are disjoint. Results are bitwise reproducible for the
 * same entry point and shape (the launch shape, and so the rounding order,
 * depends on the mode and the sizes only).
 *
 * Errors: a negative status is returned and nothing is launched when an
 * argument is invalid; PA_EHIP reports a failed launch. Data errors are
 * undefined results but never out-of-bounds accesses: a context longer than
 * max_blocks_per_seq * 16 is cut to that length, and a table entry outside
 * [0, num_blocks) is read as block 0 (both raise a bit in err_flag when the
 * debug entry point is given one). A sequence with seq_len <= 0 gets a zero
 * output; an empty batch (num_seqs == 0) is a no-op and its pointers may be
 * NULL. Slots beyond a context (tail slots of its last block, padding table
 * entries, unreferenced blocks) are never read into the result, whatever they
 * hold (NaN or Inf included).
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type shared by q, the caches and out. [prefix-doc] model attention
 * shapes: the served model runs its attention in fp16 or bf16; f32 is the
 * exact-arithmetic variant. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_F16 = 2 } pa_dtype;

/* Path selection for pa_decode_partitions / pa_lse_reduce. */
typedef enum {
  PA_MODE_AUTO = 0, /* per sequence: seq_len > 8192 -> V2, else V1 ([cd0d9e1a] rewrite, item 2) */
  PA_MODE_V1 = 1,   /* every sequence in one pass over its whole context */
  PA_MODE_V2 = 2    /* every sequence in partitions (512 tokens) + log-sum-exp reduce */
} pa_mode;

typedef struct {
  int32_t num_seqs;           /* S  >= 0 */
  int32_t num_heads;          /* H  >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv >= 1; H / Hkv must be 1..16 */
  int32_t head_dim;           /* D: 128 or 256 ([prefix-doc] model attention shapes) */
  int32_t block_size;         /* tokens per physical block: must be 16 */
  int32_t max_blocks_per_seq; /* table width (>= 1) */
  int64_t num_blocks;         /* pool size (>= 1) */
  int32_t dtype;              /* pa_dtype */
  int32_t partition_size;     /* tokens per V2 partition: 0 (= PA_PARTITION_SIZE, 512) or 256.
                               * [prefix-doc] partition-size note: both sizes existed
                               * before 512 was made the one size; 256 is opt-in here.
                               * It changes the partials' layout (Pmax) and the
                               * rounding order, not the definition. The V1/V2
                               * threshold stays 8192 tokens. */
} pa_shape;

enum {
  PA_OK = 0,
  PA_EINVAL = -1,       /* null pointer, negative or inconsistent size, H % Hkv != 0 */
  PA_EUNSUPPORTED = -2, /* D not 128/256, block_size != 16, G > 16, unknown dtype/mode,
                         partition_size not 0/256/512 */
  PA_EALIGN = -3,       /* a pointer is not 16-byte aligned */
  PA_EHIP = -4,         /* the HIP launch failed */
  PA_ESCRATCH = -5      /* pa_decode_noalloc: the partials do not fit the library's scratch */
};

#define PA_BLOCK_SIZE 16
#define PA_PARTITION_SIZE 512 /* [cd0d9e1a] V2 implementation; [prefix-doc] partition-size note */
#define PA_PARTITION_SIZE_SMALL 256 /* the opt-in alternative (pa_shape.partition_size) */
#define PA_V2_THRESHOLD 8192  /* [cd0d9e1a] rewrite, item 2 */

/* Single pass over every sequence's whole context ([cd0d9e1a] V1 discussion
 * in "V2 implementation"). Writes out. */
int pa_decode_v1(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                 float scale, void* stream);

/* Two phases for every sequence ([cd0d9e1a] V2 implementation): phase 1
 * writes per-partition max_logits (natural-log units of the scaled logits),
 * exp_sums (relative to that max) and tmp_out (normalised by its exp_sum) for
 * p < ceil(seq_len / PS) (PS = 512, or 256 when the shape opts in); phase 2
 * combines them into out. */
int pa_decode_v2(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                 float scale, float* exp_sums, float* max_logits, float* tmp_out, void* stream);

/* Per-sequence choice ([cd0d9e1a] rewrite, item 2): seq_len > 8192 takes the
 * two-phase path, the others the single pass, in one launch per phase and with
 * no host synchronisation. Partials are written for the long sequences only. */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
              float scale, float* exp_sums, float* max_logits, float* tmp_out, void* stream);

/* pa_decode without caller buffers and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same kernels, launch
 * shapes and results as pa_decode (bitwise); the partials live in one
 * library-owned device array of PA_NOALLOC_SCRATCH_BYTES per GPU, kept until
 * the process ends (its address is looked up once per device, on the first
 * call there).
 *   Limit: S * H * Pmax * (D + 2) floats (plus alignment) must fit; larger
 *   shapes return PA_ESCRATCH before anything is launched. 64 MiB holds, at
 *   16 heads and head_dim 128, the partials of 20 sequences of 100K tokens.
 *   Nothing in the array needs to start at zero: every partial the reduce
 *   reads is written earlier in the same call.
 *   Calls that overlap on one GPU (different streams, or threads without
 *   ordering) share that array and race; calls ordered on one stream do not.
 * Arguments, layouts and the other errors as for pa_decode. */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                      float scale, void* stream);

/* Phase 1 alone under `mode`: single-pass sequences write out, partitioned
 * ones write partials. pa_decode = pa_decode_partitions(AUTO) +
 * pa_lse_reduce(AUTO). Partial buffers may be NULL when mode is PA_MODE_V1. */
int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const pa_shape* shape, float scale, float* exp_sums, float* max_logits,
                         float* tmp_out, int mode, void* stream);

/* Phase 2 alone ([cd0d9e1a] V2 implementation, phase 2): for each sequence
 * the mode sends to V2 (every sequence under PA_MODE_V2, seq_len > 8192 under
 * PA_MODE_AUTO), M = max_p max_logits, c_p = exp(max_logits_p - M) *
 * exp_sums_p, out = sum_p c_p tmp_out_p / sum_p c_p over p < ceil(seq_len/PS).
 * Other sequences' out rows are left untouched. */
int pa_lse_reduce(void* out, const float* exp_sums, const float* max_logits, const float* tmp_out,
                  const int32_t* seq_lens, const pa_shape* shape, int mode, void* stream);

/* Debug form of pa_decode_partitions: also writes gather_trace[s][i] = the
 * physical block id the kernel loaded for logical block i of sequence s
 * (entries it did not load are left as they were), and ORs 1 into *err_flag
 * for a context cut to the table width, 2 for an out-of-range block id.
 * gather_trace is int32 [S, max_blocks_per_seq]; either pointer may be NULL. */
int pa_decode_partitions_debug(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               const pa_shape* shape, float scale, float* exp_sums,
                               float* max_logits, float* tmp_out, int mode,
                               int32_t* gather_trace, int32_t* err_flag, void* stream);

/* Measurement forms of pa_decode_partitions and pa_lse_reduce: the kernel is
 * launched with start_event recorded as it begins and stop_event as it ends
 * (hipEvent_t handles created by the caller; either may be NULL), so the
 * pair times that kernel alone, on `stream`. When there is nothing to launch
 * (an empty batch, or PA_MODE_V1 for the reduce) both events are recorded
 * back to back on `stream`, so the pair still completes. */
int pa_decode_partitions_timed(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               const pa_shape* shape, float scale, float* exp_sums,
                               float* max_logits, float* tmp_out, int mode, void* start_event,
                               void* stop_event, void* stream);
int pa_lse_reduce_timed(void* out, const float* exp_sums, const float* max_logits, const float* tmp_out,
                        const int32_t* seq_lens, const pa_shape* shape, int mode, void* start_event,
                        void* stop_event, void* stream);

/* Prefix / chunked-prefill attention over the same paged cache ([cd0d9e1a]
 * "paged_attn.py rewrite" item 1: the prefix path gathers the context's K/V
 * from the cache and walks query tiles over it with the online softmax;
 * [prefix-doc]: query tiles against key/value tiles, head_dim 128/256, GQA,
 * fp16/bf16, chunked prefill).
 *
 * Sequence s holds seq_lens[s] = L tokens in the cache; the last
 * Q = query_start_loc[s+1] - query_start_loc[s] of them are the chunk being
 * prefilled, their K/V already written to the cache. Chunk token i
 * (0 <= i < Q) sits at position L - Q + i and attends to cache tokens
 * 0 .. L - Q + i (its prefix, then the chunk causally); a token whose
 * position is negative (Q > L) gets a zero output.
 *
 *   q, out           [num_query_tokens, H, D]  dtype (bf16 or fp16 only),
 *                    packed by token: rows query_start_loc[s] .. [s+1]-1
 *                    belong to sequence s
 *   query_start_loc  int32 [S + 1], non-decreasing, [0] = 0,
 *                    [S] = num_query_tokens
 *   max_query_len    >= every Q (sizes the grid; host value, no device read)
 *   k_cache, v_cache, block_tables, seq_lens as for decode; shape.dtype must
 *   be PA_BF16 or PA_F16 (PA_EUNSUPPORTED otherwise); partition_size unused.
 *
 * Returns PA_OK with nothing launched when num_seqs, num_query_tokens or
 * max_query_len is 0. Data errors are undefined results, never out-of-bounds
 * accesses: query_start_loc entries are clamped to [0, num_query_tokens],
 * seq_lens to [0, max_blocks_per_seq * 16], out-of-range block ids read block
 * 0; chunk tokens beyond max_query_len are not computed. Bitwise
 * reproducible for the same shape. */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
               const int32_t* seq_lens, const int32_t* query_start_loc, const pa_shape* shape,
               int32_t num_query_tokens, int32_t max_query_len, float scale, void* stream);

/* Pmax = ceil(max_blocks_per_seq * 16 / PS), or a negative status. */
int64_t pa_max_partitions(const pa_shape* shape);

/* Element counts of the partial buffers: which = 0 for exp_sums and
 * max_logits (S * H * Pmax), 1 for tmp_out (S * H * Pmax * D). */
int64_t pa_partials_elems(const pa_shape* shape, int which);

/* Validation only (no launch): the status pa_decode would return for these
 * pointers and this shape. */
int pa_check_args(const void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                  const float* exp_sums, const float* max_logits, const float* tmp_out, int mode);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Library version, for the binding's load check. */
int pa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_DECODE_H */
