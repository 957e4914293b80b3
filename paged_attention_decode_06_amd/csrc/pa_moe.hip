// MoE routing path for gfx950 (MI355X): router top-k softmax, stable sort of
// the token-expert pairs by expert, gather of the expert inputs into sorted
// order, and the weighted scatter-back of the expert outputs.
//
// Method (project_6 commit cd0d9e1a, qwen3_6_scripts, the MoE prefill
// rewrite; project_6 commit 490ff98a, Dockerfile, topk_softmax): flatten the
// T x K assignments, sort them by expert so every expert's rows are
// contiguous, and add the weighted expert outputs back in one pass. The
// expert GEMMs between permute and combine are not part of this file.
//
// Design (wave64):
//   * top-k softmax: one wave per token, E/64 logits per lane; max and sum by
//     DPP reductions, then K rounds of (wave max of the untaken logits, the
//     lowest id holding it by ballots).
//   * sort: a stable counting sort. Chunks of 1024 pairs: every pair's rank
//     among the earlier same-expert pairs of its chunk (wave ballots, then a
//     prefix over the chunk's waves) and the chunk's per-expert counts; a
//     scan over chunks per expert; the expert offsets; then every pair lands
//     at offset + earlier chunks' count + rank. Four launches, or one
//     workgroup walking the chunks in order for up to 8192 pairs.
//   * permute and combine: one wave per row, 16-byte loads and stores; the
//     combine gathers each token's K rows (no atomics) and sums them in fp32
//     in the order j = 0..K-1.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_decode.h"
#include "pa_moe.h"

namespace {

constexpr int kSortChunk = 1024;   // pairs per counting-sort chunk (one thread each)
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Rows read once carry the non-temporal hint: with four 1 KB slices per
// combine pass, measured 117.7 -> 104.4 us for the combine at 16384 tokens x
// top 8 x 2048 bf16. Stores stay plain: non-temporal stores made the
// permute's scattered row writes slower (126 against 90 us, same workload).
__device__ __forceinline__ u32x4 ld_rows(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------- top-k softmax
// Wave-wide reductions on DPP lane moves (no LDS crossbar): swaps within
// quads, mirrors within half rows and rows, then the row broadcasts that
// fold rows 0-2 into row 3; lane 63 ends with the result, read back as a
// uniform value. The combining order is fixed, so sums are reproducible.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float v) {  // lanes outside ROWS keep v
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                               CTRL, ROWS, 0xf, false));
}

template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
  x = op(x, dpp_move<0xb1, 0xf>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_move<0x4e, 0xf>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_move<0x141, 0xf>(x));  // row_half_mirror
  x = op(x, dpp_move<0x140, 0xf>(x));  // row_mirror: every lane holds its row's result
  x = op(x, dpp_move<0x142, 0xa>(x));  // row_bcast:15 into rows 1 and 3
  x = op(x, dpp_move<0x143, 0xc>(x));  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce(x, [](float a, float b) { return a + b; });
}

// Reductions over the 16 lanes of a DPP row (every lane gets the result):
// swaps within quads, then the half-row and row mirrors.
template <typename Op>
__device__ __forceinline__ float row16_reduce(float x, Op op) {
  x = op(x, dpp_move<0xb1, 0xf>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_move<0x4e, 0xf>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_move<0x141, 0xf>(x));  // row_half_mirror
  return op(x, dpp_move<0x140, 0xf>(x));  // row_mirror
}
__device__ __forceinline__ int row16_min(int x) {
  const float r = row16_reduce(__builtin_bit_cast(float, x), [](float a, float b) {
    return __builtin_bit_cast(float, min(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b)));
  });
  return __builtin_bit_cast(int, r);
}

// Sixteen lanes per token (four tokens per wave) for E <= 256 and K <= 16:
// lane s of a row holds logits s, s + 16, ... (V = E/16 rounded up to a
// power of two). Round j: the row maximum of the untaken logits, then the
// lowest expert id holding it (each lane's lowest candidate, then the row
// minimum); the owner lane marks it taken in a bit mask. Same results as
// the one-wave-per-token kernel below (ties to the lower id, NaN never
// chosen), with 4 instead of 7 reduction steps per round plus a readlane
// and four tokens per wave: 22.2 -> 17.8 us at 16384 tokens x 256 experts x
// top 8. Each lane walks V logits per round, so with few tokens (a wave
// each, latency-bound) the one-wave kernel is faster: 5.5 against 8.0 us at
// 256 tokens; the row kernel takes batches of kTopkRowTokens and more.
constexpr int kTopkRowTokens = 4096;
template <int V>
__global__ __launch_bounds__(kThreads) void moe_topk_softmax_row16_kernel(float* __restrict__ w_out,
                                                                          int32_t* __restrict__ id_out,
                                                                          const float* __restrict__ logits,
                                                                          int T, int E, int K, int renorm) {
  static_assert(V <= 16, "taken bits fit one 32-bit mask");
  const int lane = threadIdx.x & 63, s = lane & 15;
  const int t = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool live = t < T;  // rows of a wave past T compute on a copy of row T - 1 and store nothing
  const float* row = logits + (int64_t)(live ? t : T - 1) * E;
  float v[V];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int e = 16 * u + s;
    v[u] = e < E ? row[e] : -INFINITY;
  }
  float m = v[0];
#pragma unroll
  for (int u = 1; u < V; ++u) m = fmaxf(m, v[u]);
  m = row16_reduce(m, [](float a, float b) { return fmaxf(a, b); });
  float part = 0.f;
#pragma unroll
  for (int u = 0; u < V; ++u)
    if (16 * u + s < E) part += __builtin_amdgcn_exp2f((v[u] - m) * kLog2e);
  const float sum = row16_reduce(part, [](float a, float b) { return a + b; });

  uint32_t avail = 0;  // bit u: logit 16u + s exists, is not NaN and is not taken
#pragma unroll
  for (int u = 0; u < V; ++u)
    if (16 * u + s < E && !(v[u] != v[u])) avail |= 1u << u;
  float my_w = 0.f;
  int my_id = 0;
  for (int j = 0; j < K; ++j) {
    float lm = -INFINITY;
#pragma unroll
    for (int u = 0; u < V; ++u)
      if ((avail >> u) & 1u) lm = fmaxf(lm, v[u]);
    const float best = row16_reduce(lm, [](float a, float b) { return fmaxf(a, b); });
    int cand = 0x7fffffff;
#pragma unroll
    for (int u = V - 1; u >= 0; --u)
      if (((avail >> u) & 1u) && v[u] == best) cand = 16 * u + s;
    int id = row16_min(cand);
    if (id == 0x7fffffff) {
      id = 0;  // nothing left but NaN logits: a data error, kept in range
    } else if ((id & 15) == s) {
      avail &= ~(1u << (id >> 4));
    }
    if (s == j) {
      my_w = best > -INFINITY ? __builtin_amdgcn_exp2f((best - m) * kLog2e) / sum : 0.f;
      my_id = id;
    }
  }
  if (renorm) {
    const float tot = row16_reduce(s < K ? my_w : 0.f, [](float a, float b) { return a + b; });
    if (tot > 0.f) my_w /= tot;
  }
  if (live && s < K) {
    w_out[(int64_t)t * K + s] = my_w;
    id_out[(int64_t)t * K + s] = my_id;
  }
}

// One wave per token. Round j: the wave maximum of the logits not yet taken
// (DPP reduction), then the lowest expert id holding it: for u = 0, 1, ...
// the ballot of lanes whose u-th logit is that maximum and untaken; the first
// non-empty ballot's lowest lane wins (id = lane + 64u).
template <int VPL>
__global__ __launch_bounds__(kThreads) void moe_topk_softmax_kernel(float* __restrict__ w_out,
                                                                    int32_t* __restrict__ id_out,
                                                                    const float* __restrict__ logits, int T,
                                                                    int E, int K, int renorm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float v[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    const int e = lane + 64 * u;
    v[u] = e < E ? row[e] : -INFINITY;
  }
  float m = v[0];
#pragma unroll
  for (int u = 1; u < VPL; ++u) m = fmaxf(m, v[u]);
  m = wave_max(m);
  float part = 0.f;
#pragma unroll
  for (int u = 0; u < VPL; ++u)
    if (lane + 64 * u < E) part += __builtin_amdgcn_exp2f((v[u] - m) * kLog2e);
  const float sum = wave_sum(part);

  bool avail[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) avail[u] = lane + 64 * u < E && !(v[u] != v[u]);  // NaN never chosen
  float my_w = 0.f;
  int my_id = 0;
  for (int j = 0; j < K; ++j) {
    float lm = -INFINITY;
#pragma unroll
    for (int u = 0; u < VPL; ++u)
      if (avail[u]) lm = fmaxf(lm, v[u]);
    const float best = wave_max(lm);
    int id = -1;
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      if (id < 0) {
        const uint64_t hit = __builtin_amdgcn_ballot_w64(avail[u] && v[u] == best);
        if (hit) {
          const int l = __builtin_ctzll(hit);
          id = l + 64 * u;
          if (lane == l) avail[u] = false;
        }
      }
    }
    if (id < 0) id = 0;  // nothing left but NaN logits: a data error, kept in range
    if (lane == j) {
      my_w = (id >= 0 && best > -INFINITY) ? __builtin_amdgcn_exp2f((best - m) * kLog2e) / sum : 0.f;
      my_id = id;
    }
  }
  if (renorm) {
    const float s = wave_sum(lane < K ? my_w : 0.f);
    if (s > 0.f) my_w /= s;
  }
  if (lane < K) {
    w_out[(int64_t)t * K + lane] = my_w;
    id_out[(int64_t)t * K + lane] = my_id;
  }
}

// ---------------------------------------------------------------- stable counting sort
// Phase 1, one workgroup per chunk of 1024 pairs (16 waves of 64 consecutive
// pairs): each wave ranks its pairs among the earlier same-expert pairs of the
// wave (the mask of lanes holding the same expert, the count of its set bits
// below each lane) and counts them per expert; a prefix over the 16 waves per
// expert turns that into the rank within the chunk and the chunk's per-expert
// counts.
constexpr int kSortWaves = kSortChunk / 64;
static_assert(PA_MOE_MAX_EXPERTS <= 1024, "expert ids are matched on at most 10 bits");

// Rank of each valid lane's expert e among the lower lanes of the wave that
// hold the same expert; the lowest such lane stores the wave's count of e in
// wcnt_row[e]. The lanes sharing e are found bit by bit: one ballot per bit
// of the expert id (the bits of E - 1, at most 10), each lane keeping the
// lanes that agree with it on that bit, so the cost does not depend on how
// many distinct experts the wave holds.
template <typename C>
__device__ __forceinline__ int rank_in_wave(int e, bool valid, int lane, int ebits, C* wcnt_row) {
  uint64_t m = __builtin_amdgcn_ballot_w64(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {
    if (b < ebits) {
      const bool bit = ((e >> b) & 1) != 0;
      const uint64_t mb = __builtin_amdgcn_ballot_w64(bit);
      m &= bit ? mb : ~mb;
    }
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rw = __builtin_popcountll(m & below);
  if (valid && rw == 0) wcnt_row[e] = (C)__builtin_popcountll(m);
  return rw;
}

__device__ __forceinline__ int expert_bits(int E) { return E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0; }

__global__ __launch_bounds__(kSortChunk) void moe_sort_count_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                                    int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ rank) {
  extern __shared__ int32_t wcnt[];  // [kSortWaves][E]
  const int c = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int a = c * kSortChunk + t;
  const bool valid = a < N;
  const int e = valid ? clampi(ids[a], 0, E - 1) : -1;
  for (int i = t; i < kSortWaves * E; i += kSortChunk) wcnt[i] = 0;
  __syncthreads();
  const int rw = rank_in_wave(e, valid, lane, expert_bits(E), wcnt + w * E);
  __syncthreads();
  if (t < E) {
    int run = 0;
#pragma unroll
    for (int i = 0; i < kSortWaves; ++i) {
      const int x = wcnt[i * E + t];
      wcnt[i * E + t] = run;
      run += x;
    }
    counts[(int64_t)c * E + t] = run;
  }
  __syncthreads();
  if (valid) rank[a] = wcnt[w * E + e] + rw;
}

// Phase 2, one workgroup per expert: counts[c][e] becomes the number of
// expert-e pairs in chunks before c (a block-wide exclusive scan over the
// chunks, 256 at a time), and totals[e] the expert's pair count.
__global__ __launch_bounds__(kThreads) void moe_sort_colscan_kernel(int32_t* __restrict__ counts, int NC, int E,
                                                                    int32_t* __restrict__ totals) {
  __shared__ int32_t sc[kThreads];
  const int e = blockIdx.x, t = threadIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < NC; c0 += kThreads) {
    const int c = c0 + t;
    const int x = c < NC ? counts[(int64_t)c * E + e] : 0;
    sc[t] = x;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {  // inclusive Hillis-Steele scan
      const int add = t >= d ? sc[t - d] : 0;
      __syncthreads();
      sc[t] += add;
      __syncthreads();
    }
    if (c < NC) counts[(int64_t)c * E + e] = carry + sc[t] - x;
    carry += sc[kThreads - 1];
    __syncthreads();
  }
  if (t == 0) totals[e] = carry;
}

// Phase 3 (one workgroup): expert offsets = exclusive scan of the totals.
__global__ __launch_bounds__(PA_MOE_MAX_EXPERTS) void moe_sort_offsets_kernel(const int32_t* __restrict__ totals,
                                                                              int E, int N,
                                                                              int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[PA_MOE_MAX_EXPERTS];
  const int e = threadIdx.x;
  const int x = (e < E && totals) ? totals[e] : 0;
  tot[e] = x;
  __syncthreads();
  for (int d = 1; d < PA_MOE_MAX_EXPERTS; d <<= 1) {
    const int add = e >= d ? tot[e - d] : 0;
    __syncthreads();
    tot[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e] = tot[e] - x;
  if (e == 0) offsets[E] = N;
}

// Phase 4: every pair lands at its expert's offset, plus the same-expert
// pairs of earlier chunks, plus its rank within its chunk.
__global__ __launch_bounds__(kSortChunk) void moe_sort_scatter_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                                      const int32_t* __restrict__ counts,
                                                                      const int32_t* __restrict__ rank,
                                                                      const int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ sorted_pairs,
                                                                      int32_t* __restrict__ pair_pos) {
  const int c = blockIdx.x;
  const int a = c * kSortChunk + threadIdx.x;
  if (a < N) {
    const int e = clampi(ids[a], 0, E - 1);
    const int pos = offsets[e] + counts[(int64_t)c * E + e] + rank[a];
    sorted_pairs[pos] = a;
    pair_pos[a] = pos;
  }
}

// Small pair sets (up to kSortSmallChunks chunks), one workgroup, one launch:
// the same per-chunk ranks, chunk after chunk, with each expert's running
// count of the earlier chunks kept in LDS; then the offsets scan and the
// scatter. Same result as the four-launch path.
constexpr int kSortSmallChunks = 4;
static_assert(kSortSmallChunks <= 8, "the single-workgroup sort is instantiated for up to 8 chunks");

template <int R>
__global__ __launch_bounds__(kSortChunk) void moe_sort_small_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                                    int32_t* __restrict__ sorted_pairs,
                                                                    int32_t* __restrict__ pair_pos,
                                                                    int32_t* __restrict__ offsets) {
  static_assert(kSortChunk == PA_MOE_MAX_EXPERTS, "one thread per expert in the scans");
  __shared__ uint16_t wcnt[kSortWaves * PA_MOE_MAX_EXPERTS];  // per-wave counts of one chunk (<= 64 each)
  __shared__ int32_t run[PA_MOE_MAX_EXPERTS];                 // pairs of each expert in earlier chunks
  __shared__ int32_t scan[PA_MOE_MAX_EXPERTS];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int e[R], rk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int a = r * kSortChunk + t;
    e[r] = a < N ? clampi(ids[a], 0, E - 1) : -1;
  }
  run[t] = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    for (int i = t; i < kSortWaves * E; i += kSortChunk) wcnt[i] = 0;
    __syncthreads();
    const int rw = rank_in_wave(e[r], e[r] >= 0, lane, expert_bits(E), wcnt + w * E);
    __syncthreads();
    int chunk_total = 0;
    if (t < E) {  // exclusive prefix over the chunk's waves, per expert
#pragma unroll
      for (int i = 0; i < kSortWaves; ++i) {
        const int x = wcnt[i * E + t];
        wcnt[i * E + t] = (uint16_t)chunk_total;
        chunk_total += x;
      }
    }
    __syncthreads();
    rk[r] = e[r] >= 0 ? run[e[r]] + wcnt[w * E + e[r]] + rw : 0;
    __syncthreads();
    if (t < E) run[t] += chunk_total;
  }
  __syncthreads();
  const int x = t < E ? run[t] : 0;
  scan[t] = x;
  __syncthreads();
  for (int d = 1; d < PA_MOE_MAX_EXPERTS; d <<= 1) {
    const int add = t >= d ? scan[t - d] : 0;
    __syncthreads();
    scan[t] += add;
    __syncthreads();
  }
  const int off = scan[t] - x;
  if (t < E) {
    offsets[t] = off;
    run[t] = off;
  }
  if (t == 0) offsets[E] = N;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int a = r * kSortChunk + t;
    if (a < N) {
      const int pos = run[e[r]] + rk[r];
      sorted_pairs[pos] = a;
      pair_pos[a] = pos;
    }
  }
}

// ---------------------------------------------------------------- permute / combine
// Token-major scatter: a wave reads token t's row once and writes it to the
// K sorted positions of t's pairs. Every row of x is read from HBM once and
// every sorted row written once, so the traffic is the algorithmic minimum
// (the gather form, a wave per sorted row, re-read each token row K times
// through the caches and ran at 3.6 TB/s of writes against 6.5 for a plain
// fill).
// Token-major scatter: a wave reads token t's row once and writes it to the
// K sorted positions of t's pairs, so every row of x leaves HBM once. The
// gather form (a wave per sorted row) re-read each token row K times through
// the caches: 150 us against 124 us for this form at 16384 tokens x top 8 x
// 2048 bf16. Two or four tokens per wave measured the same as one.
__global__ __launch_bounds__(kThreads) void moe_permute_kernel(char* __restrict__ dst, const char* __restrict__ src,
                                                               const int32_t* __restrict__ pair_pos, int T, int K,
                                                               int64_t row_bytes) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int N = T * K;
  const int my_pos = lane < K ? clampi(pair_pos[(int64_t)t * K + lane], 0, N - 1) : 0;
  const char* s = src + (int64_t)t * row_bytes;
  // four 1 KB slices per pass: the loads, then K copies of them
  for (int64_t off0 = (int64_t)lane * 16; off0 < row_bytes; off0 += 4 * 64 * 16) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t off = off0 + (int64_t)u * 64 * 16;
      if (off < row_bytes) v[u] = ld_rows(s + off);
    }
    for (int j = 0; j < K; ++j) {
      char* d = dst + (int64_t)__builtin_amdgcn_readlane(my_pos, j) * row_bytes;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t off = off0 + (int64_t)u * 64 * 16;
        if (off < row_bytes) *reinterpret_cast<u32x4*>(d + off) = v[u];
      }
    }
  }
}

template <typename E>
struct Row16;  // 16 raw bytes of a row <-> floats
template <>
struct Row16<float> {
  static constexpr int n = 4;
  typedef float f4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ void unpack(float (&f)[8], u32x4 x) {
    const f4 v = __builtin_bit_cast(f4, x);  // whole-vector casts only
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
  }
  static __device__ __forceinline__ u32x4 pack(const float (&f)[8]) {
    const f4 v = {f[0], f[1], f[2], f[3]};
    return __builtin_bit_cast(u32x4, v);
  }
};
template <typename H>
struct Row16Half {
  static constexpr int n = 8;
  typedef H h8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ void unpack(float (&f)[8], u32x4 x) {
    const h8 h = __builtin_bit_cast(h8, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  }
  static __device__ __forceinline__ u32x4 pack(const float (&f)[8]) {
    h8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (H)f[i];
    return __builtin_bit_cast(u32x4, h);
  }
};
template <>
struct Row16<__bf16> : Row16Half<__bf16> {};
template <>
struct Row16<_Float16> : Row16Half<_Float16> {};

// One wave per token. Each pass covers kCombineU 1 KB slices of the row and
// issues the loads of up to 8 choices for all of them before any arithmetic,
// so a wave keeps 16 loads of 16 bytes in flight; the sum still runs in the
// order j = 0..K-1 for every element.
constexpr int kCombineU = 4;

template <typename E>
__global__ __launch_bounds__(kThreads) void moe_combine_kernel(char* __restrict__ out, const char* __restrict__ y,
                                                               const float* __restrict__ weights,
                                                               const int32_t* __restrict__ pair_pos, int T, int K,
                                                               int64_t row_bytes) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int N = T * K;
  // lane j < K holds choice j's weight and row; broadcast below in order j.
  float wl = 0.f;
  int pl = 0;
  if (lane < K) {
    wl = weights[(int64_t)t * K + lane];
    pl = clampi(pair_pos[(int64_t)t * K + lane], 0, N - 1);
  }
  for (int64_t off0 = (int64_t)lane * 16; off0 < row_bytes; off0 += kCombineU * 64 * 16) {
    float acc[kCombineU][8];
#pragma unroll
    for (int u = 0; u < kCombineU; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
    for (int j0 = 0; j0 < K; j0 += 8) {
      u32x4 buf[8][kCombineU];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int pj = __shfl(pl, j0 + jj);
#pragma unroll
        for (int u = 0; u < kCombineU; ++u) {
          const int64_t off = off0 + (int64_t)u * 64 * 16;
          buf[jj][u] = (j0 + jj < K && off < row_bytes)
                           ? ld_rows(y + (int64_t)pj * row_bytes + off)
                           : (u32x4){0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float wj = __shfl(wl, j0 + jj);
        if (j0 + jj < K) {
#pragma unroll
          for (int u = 0; u < kCombineU; ++u) {
            float f[8];
            Row16<E>::unpack(f, buf[jj][u]);
#pragma unroll
            for (int i = 0; i < Row16<E>::n; ++i) acc[u][i] += wj * f[i];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineU; ++u) {
      const int64_t off = off0 + (int64_t)u * 64 * 16;
      if (off < row_bytes) *reinterpret_cast<u32x4*>(out + (int64_t)t * row_bytes + off) = Row16<E>::pack(acc[u]);
    }
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_bytes(int dtype) {
  return dtype == PA_F32 ? 4 : (dtype == PA_BF16 || dtype == PA_F16) ? 2 : 0;
}

int check_tek(int32_t T, int32_t E, int32_t K) {
  if (T < 0 || E < 1 || K < 1) return PA_EINVAL;
  if (E > PA_MOE_MAX_EXPERTS || K > PA_MOE_MAX_TOPK || K > E) return PA_EUNSUPPORTED;
  if ((int64_t)T * K >= ((int64_t)1 << 31) - kSortChunk) return PA_EUNSUPPORTED;
  return PA_OK;
}

int check_rows(int32_t T, int32_t K, int32_t hidden, int32_t dtype) {
  if (T < 0 || K < 1 || hidden < 1) return PA_EINVAL;
  if (K > PA_MOE_MAX_TOPK) return PA_EUNSUPPORTED;
  const int eb = elem_bytes(dtype);
  if (!eb) return PA_EUNSUPPORTED;
  if (((int64_t)hidden * eb) % 16) return PA_EALIGN;
  if ((int64_t)T * K >= ((int64_t)1 << 31)) return PA_EUNSUPPORTED;
  return PA_OK;
}

hipError_t finish() { return hipGetLastError(); }

}  // namespace

extern "C" {

int pa_moe_topk_softmax(float* topk_weights, int32_t* topk_ids, const float* logits, int32_t T, int32_t E,
                        int32_t K, int renormalize, void* stream) {
  const int st = check_tek(T, E, K);
  if (st != PA_OK) return st;
  if (T == 0) return PA_OK;
  if (!topk_weights || !topk_ids || !logits) return PA_EINVAL;
  if (!aligned(topk_weights, 4) || !aligned(topk_ids, 4) || !aligned(logits, 4)) return PA_EALIGN;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  if (E <= 256 && K <= 16 && T >= kTopkRowTokens) {
    const dim3 grid16((unsigned)((T + 15) / 16)), block16(kThreads);
    const int v16 = (E + 15) / 16;
    if (v16 <= 1) hipLaunchKernelGGL(moe_topk_softmax_row16_kernel<1>, grid16, block16, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
    else if (v16 <= 2) hipLaunchKernelGGL(moe_topk_softmax_row16_kernel<2>, grid16, block16, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
    else if (v16 <= 4) hipLaunchKernelGGL(moe_topk_softmax_row16_kernel<4>, grid16, block16, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
    else if (v16 <= 8) hipLaunchKernelGGL(moe_topk_softmax_row16_kernel<8>, grid16, block16, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
    else hipLaunchKernelGGL(moe_topk_softmax_row16_kernel<16>, grid16, block16, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
    return finish() == hipSuccess ? PA_OK : PA_EHIP;
  }
  const dim3 grid((unsigned)((T + 3) / 4)), block(kThreads);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1) hipLaunchKernelGGL(moe_topk_softmax_kernel<1>, grid, block, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
  else if (vpl <= 2) hipLaunchKernelGGL(moe_topk_softmax_kernel<2>, grid, block, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
  else if (vpl <= 4) hipLaunchKernelGGL(moe_topk_softmax_kernel<4>, grid, block, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
  else if (vpl <= 8) hipLaunchKernelGGL(moe_topk_softmax_kernel<8>, grid, block, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
  else hipLaunchKernelGGL(moe_topk_softmax_kernel<16>, grid, block, 0, s, topk_weights, topk_ids, logits, T, E, K, renormalize);
  return finish() == hipSuccess ? PA_OK : PA_EHIP;
}

int64_t pa_moe_sort_workspace_bytes(int32_t T, int32_t E, int32_t K) {
  const int st = check_tek(T, E, K);
  if (st != PA_OK) return st;
  const int64_t N = (int64_t)T * K;
  const int64_t NC = (N + kSortChunk - 1) / kSortChunk;
  return (NC * E + N + E) * (int64_t)sizeof(int32_t);
}

int pa_moe_sort_by_expert(int32_t* sorted_pairs, int32_t* pair_pos, int32_t* expert_offsets,
                          const int32_t* topk_ids, int32_t T, int32_t E, int32_t K, void* workspace,
                          int64_t workspace_bytes, void* stream) {
  const int st = check_tek(T, E, K);
  if (st != PA_OK) return st;
  if (!expert_offsets) return PA_EINVAL;
  if (!aligned(expert_offsets, 4)) return PA_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int N = T * K;
  if (N == 0) {  // every expert's range is empty: zero offsets from the offsets scan alone
    (void)hipGetLastError();
    hipLaunchKernelGGL(moe_sort_offsets_kernel, dim3(1), dim3(PA_MOE_MAX_EXPERTS), 0, s, nullptr, E, 0,
                       expert_offsets);
    return finish() == hipSuccess ? PA_OK : PA_EHIP;
  }
  if (!sorted_pairs || !pair_pos || !topk_ids || !workspace) return PA_EINVAL;
  if (!aligned(sorted_pairs, 4) || !aligned(pair_pos, 4) || !aligned(topk_ids, 4) || !aligned(workspace, 4))
    return PA_EALIGN;
  if (workspace_bytes < pa_moe_sort_workspace_bytes(T, E, K)) return PA_EINVAL;
  const int NC = (N + kSortChunk - 1) / kSortChunk;
  if (NC <= kSortSmallChunks) {
    (void)hipGetLastError();
    const dim3 g(1), b(kSortChunk);
    if (NC <= 1) hipLaunchKernelGGL(moe_sort_small_kernel<1>, g, b, 0, s, topk_ids, N, E, sorted_pairs, pair_pos, expert_offsets);
    else if (NC <= 2) hipLaunchKernelGGL(moe_sort_small_kernel<2>, g, b, 0, s, topk_ids, N, E, sorted_pairs, pair_pos, expert_offsets);
    else if (NC <= 4) hipLaunchKernelGGL(moe_sort_small_kernel<4>, g, b, 0, s, topk_ids, N, E, sorted_pairs, pair_pos, expert_offsets);
    else hipLaunchKernelGGL(moe_sort_small_kernel<8>, g, b, 0, s, topk_ids, N, E, sorted_pairs, pair_pos, expert_offsets);
    return finish() == hipSuccess ? PA_OK : PA_EHIP;
  }
  int32_t* counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* rank = counts + (int64_t)NC * E;
  int32_t* totals = rank + N;
  const size_t lds = (size_t)kSortWaves * E * sizeof(int32_t);  // <= 64 KB at 1024 experts
  (void)hipGetLastError();
  hipLaunchKernelGGL(moe_sort_count_kernel, dim3(NC), dim3(kSortChunk), lds, s, topk_ids, N, E, counts, rank);
  hipLaunchKernelGGL(moe_sort_colscan_kernel, dim3(E), dim3(kThreads), 0, s, counts, NC, E, totals);
  hipLaunchKernelGGL(moe_sort_offsets_kernel, dim3(1), dim3(PA_MOE_MAX_EXPERTS), 0, s, totals, E, N,
                     expert_offsets);
  hipLaunchKernelGGL(moe_sort_scatter_kernel, dim3(NC), dim3(kSortChunk), 0, s, topk_ids, N, E, counts, rank,
                     expert_offsets, sorted_pairs, pair_pos);
  return finish() == hipSuccess ? PA_OK : PA_EHIP;
}

int pa_moe_permute(void* x_sorted, const void* x, const int32_t* pair_pos, int32_t T, int32_t K, int32_t hidden,
                   int32_t dtype, void* stream) {
  const int st = check_rows(T, K, hidden, dtype);
  if (st != PA_OK) return st;
  if (T == 0) return PA_OK;
  if (!x_sorted || !x || !pair_pos) return PA_EINVAL;
  if (!aligned(x_sorted, 16) || !aligned(x, 16) || !aligned(pair_pos, 4)) return PA_EALIGN;
  const int64_t rb = (int64_t)hidden * elem_bytes(dtype);
  (void)hipGetLastError();
  hipLaunchKernelGGL(moe_permute_kernel, dim3((unsigned)((T + 3) / 4)), dim3(kThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<char*>(x_sorted), reinterpret_cast<const char*>(x), pair_pos, T, K, rb);
  return finish() == hipSuccess ? PA_OK : PA_EHIP;
}

int pa_moe_combine(void* out, const void* y_sorted, const float* topk_weights, const int32_t* pair_pos,
                   int32_t T, int32_t K, int32_t hidden, int32_t dtype, void* stream) {
  const int st = check_rows(T, K, hidden, dtype);
  if (st != PA_OK) return st;
  if (T == 0) return PA_OK;
  if (!out || !y_sorted || !topk_weights || !pair_pos) return PA_EINVAL;
  if (!aligned(out, 16) || !aligned(y_sorted, 16) || !aligned(topk_weights, 4) || !aligned(pair_pos, 4))
    return PA_EALIGN;
  const int64_t rb = (int64_t)hidden * elem_bytes(dtype);
  const dim3 grid((unsigned)((T + 3) / 4)), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  char* o = reinterpret_cast<char*>(out);
  const char* y = reinterpret_cast<const char*>(y_sorted);
  (void)hipGetLastError();
  if (dtype == PA_F32)
    hipLaunchKernelGGL(moe_combine_kernel<float>, grid, block, 0, s, o, y, topk_weights, pair_pos, T, K, rb);
  else if (dtype == PA_BF16)
    hipLaunchKernelGGL(moe_combine_kernel<__bf16>, grid, block, 0, s, o, y, topk_weights, pair_pos, T, K, rb);
  else
    hipLaunchKernelGGL(moe_combine_kernel<_Float16>, grid, block, 0, s, o, y, topk_weights, pair_pos, T, K, rb);
  return finish() == hipSuccess ? PA_OK : PA_EHIP;
}

}  // extern "C"
