// Paged-attention decode for gfx950 (MI355X): HIP kernels and the C ABI.
//
// Method (project_6 commit cd0d9e1a, qwen3_6_scripts):
//   * "paged_attn.py rewrite", item 2: a sequence whose context is longer than
//     8192 tokens takes the partitioned path (V2), the others one pass (V1).
//   * "V2 implementation": phase 1 runs attention over each 512-token
//     partition and keeps its max logit, exp-sum and output; phase 2 combines
//     partitions with log-sum-exp weights. Inside a partition the softmax is
//     the running (online) form, the same blocking flash attention uses.
//
// Kernel design (gfx950, wave64):
//   One workgroup per (sequence, KV head, partition); partition is the slowest
//   grid index so the long single-pass workgroups are dispatched first. Each
//   wave walks "tiles" of whole 16-token blocks. For a tile it
//     - loads K rows so that lane (tok = l%16, grp = l/16) holds 8 consecutive
//       head dims of token tok: the A operand of a 16x16x32 bf16 MFMA whose M
//       axis is the 16 tokens and whose N axis is the GQA group (padded to 16),
//       so one load of K serves every query head of the group;
//     - computes S[tok][g] = K q^T, leaving lane l with 4 tokens of head l%16;
//     - keeps a running max / exp-sum per head (two xor-shuffles per tile);
//     - computes O^T[d][g] += V^T[d][tok] P[tok][g]: the B operand P is the QK
//       accumulator itself (rounded to bf16), and V is loaded as whole rows
//       (16 lanes x 16 B = one 256-byte row) and transposed in registers.
//   Waves then merge (max, exp-sum, output) through LDS in a fixed order and
//   wave 0 writes either out (V1) or the three partials (V2).
//
// Data errors never turn into out-of-bounds accesses: contexts are cut to the
// table width and out-of-range block ids are read as block 0 (both reported
// through the optional error word).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_decode.h"

namespace {

constexpr int kBS = PA_BLOCK_SIZE;
constexpr int kPart = PA_PARTITION_SIZE;
constexpr int kThresh = PA_V2_THRESHOLD;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kReduceThreads = 256;
constexpr int kReduceChunk = 32;   // head dims per reduce workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  const int32_t* sl;
  void* out;
  float* exp_sums;
  float* max_logits;
  float* tmp_out;
  int32_t* trace;
  int32_t* err;
  int64_t NB;
  int S, H, Hkv, G, MB, Pmax, mode;
  float scale2;  // softmax scale times log2(e): logits are kept in base-2 units
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Work range of one workgroup. Returns 0: nothing to do, 1: attend over
// [tok_begin, tok_end), 2: single pass over an empty context (write zeros).
struct Range {
  int tok_begin, tok_end, blk_begin, blk_end;
  bool v2;
};

__device__ __forceinline__ int work_range(const Params& P, int s, int p, Range& r) {
  int L = P.sl[s];
  const int cap = P.MB * kBS;
  if (L > cap) {
    L = cap;
    if (P.err && threadIdx.x == 0) atomicOr(P.err, 1);
  }
  if (L < 0) L = 0;
  r.v2 = (P.mode == PA_MODE_V2) || (P.mode == PA_MODE_AUTO && L > kThresh);
  if (r.v2) {
    const int np = (L + kPart - 1) / kPart;
    if (p >= np) return 0;
    r.tok_begin = p * kPart;
    r.tok_end = min(r.tok_begin + kPart, L);
  } else {
    if (p != 0) return 0;
    if (L == 0) return 2;
    r.tok_begin = 0;
    r.tok_end = L;
  }
  r.blk_begin = r.tok_begin / kBS;
  r.blk_end = (r.tok_end + kBS - 1) / kBS;
  return 1;
}

// Physical block id of logical block `blk` (wave-uniform), range-checked.
template <bool TRACE>
__device__ __forceinline__ int64_t physical_block(const Params& P, const int32_t* bt_row, int s,
                                                  int blk, int lane) {
  int32_t phys = bt_row[blk];
  if ((uint64_t)(int64_t)phys >= (uint64_t)P.NB) {
    if (P.err && lane == 0) atomicOr(P.err, 2);
    phys = 0;
  }
  if (TRACE && lane == 0 && P.trace) P.trace[(int64_t)s * P.MB + blk] = phys;
  return phys;
}

// Merge the per-wave (max, exp-sum, output) triples of one workgroup into
// wave 0, in a fixed order (bitwise deterministic). acc holds the wave's
// unnormalised output for head g = lane%16 relative to its max m (base 2);
// lsum its exp-sum. On return wave 0 holds the merged values.
template <int NACC, int NW>
__device__ __forceinline__ void merge_waves(f32x4 (&acc)[NACC], float& m, float& lsum, int w,
                                            int lane, int G, float* smem) {
  if constexpr (NW > 1) {
    float* sm_m = smem;
    float* sm_l = smem + NW * 16;
    f32x4* sm_o = reinterpret_cast<f32x4*>(smem + 2 * NW * 16);
    const int g = lane & 15, grp = lane >> 4;
    if (lane < 16) {
      sm_m[w * 16 + g] = m;
      sm_l[w * 16 + g] = lsum;
    }
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) M = fmaxf(M, sm_m[i * 16 + g]);
    const float f = (m > -INFINITY) ? fast_exp2(m - M) : 0.f;
    if (w > 0 && g < G) {
      f32x4* dst = sm_o + (size_t)(w - 1) * NACC * (G * 4) + grp * G + g;
#pragma unroll
      for (int a = 0; a < NACC; ++a) dst[a * G * 4] = acc[a] * f;
    }
    __syncthreads();
    if (w == 0) {
      float lt = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const float mi = sm_m[i * 16 + g];
        lt += (mi > -INFINITY) ? sm_l[i * 16 + g] * fast_exp2(mi - M) : 0.f;
      }
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[a] *= f;
      if (g < G) {
        for (int i = 1; i < NW; ++i) {
          const f32x4* src = sm_o + (size_t)(i - 1) * NACC * (G * 4) + grp * G + g;
#pragma unroll
          for (int a = 0; a < NACC; ++a) acc[a] += src[a * G * 4];
        }
      }
      m = M;
      lsum = lt;
    }
  }
}

// Exp-sum of the wave for head lane%16: the 4 lane groups hold disjoint tokens.
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Store 4 consecutive head dims starting at dim d of head g.
template <typename T>
__device__ __forceinline__ void store4(T* row, int d, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* row, int d, f32x4 v) {
  *reinterpret_cast<f32x4*>(row + d) = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* row, int d, f32x4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 b;
  b[0] = (__bf16)v[0];
  b[1] = (__bf16)v[1];
  b[2] = (__bf16)v[2];
  b[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(row + d) = b;
}

// Final write of wave 0 after the merge. dim_of(a, i) gives the head dim the
// lane's acc[a][i] holds; dims a, a+1, a+2, a+3 (same i) are consecutive when
// `a` is a multiple of 4 (both paths below keep that property).
template <typename T, int D, int NACC, typename DimOf>
__device__ __forceinline__ void write_result(const Params& P, const Range& r, int s, int kvh,
                                             int p, int lane, const f32x4 (&acc)[NACC], float m,
                                             float lsum, DimOf dim_of) {
  const int g = lane & 15;
  if (g >= P.G) return;
  const int h = kvh * P.G + g;
  const float inv = 1.f / lsum;
  if (!r.v2) {
    T* row = reinterpret_cast<T*>(P.out) + ((int64_t)s * P.H + h) * D;
#pragma unroll
    for (int a = 0; a < NACC; a += 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v = {acc[a][i] * inv, acc[a + 1][i] * inv, acc[a + 2][i] * inv, acc[a + 3][i] * inv};
        store4<T>(row, dim_of(a, i), v);
      }
    }
  } else {
    const int64_t sh = (int64_t)s * P.H + h;
    float* row = P.tmp_out + (sh * P.Pmax + p) * D;
#pragma unroll
    for (int a = 0; a < NACC; a += 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v = {acc[a][i] * inv, acc[a + 1][i] * inv, acc[a + 2][i] * inv, acc[a + 3][i] * inv};
        store4<float>(row, dim_of(a, i), v);
      }
    }
    if (lane < 16) {
      P.exp_sums[sh * P.Pmax + p] = lsum;
      P.max_logits[sh * P.Pmax + p] = m * kLn2;  // back to natural-log units
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void write_zeros(const Params& P, int s, int kvh, int lane, int w) {
  if (w != 0) return;
  const int g = lane & 15, grp = lane >> 4;
  if (g >= P.G) return;
  T* row = reinterpret_cast<T*>(P.out) + ((int64_t)s * P.H + kvh * P.G + g) * D;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int d = grp * 4; d < D; d += 16) store4<T>(row, d, z);
}

// ---------------------------------------------------------------- bf16 path
// TB = blocks per tile. TB == 2: P.V uses the 16x16x32 MFMA over 32 tokens;
// TB == 1: the 16x16x16 MFMA over 16 tokens (fewer registers for D = 256).
template <int D, int NW, int TB, bool TRACE>
__global__ __launch_bounds__(NW * 64) void pa_partition_bf16(Params P) {
  extern __shared__ float smem[];
  constexpr int KK = D / 32;   // QK MFMAs per block (32 dims each)
  constexpr int NH = D / 128;  // 128-dim column groups of V
  constexpr int NACC = NH * 8; // output tiles: (h, j) -> dims 128h + 8m + j
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15, grp = lane >> 4;

  const int pairs = P.S * P.Hkv;
  const int pair = blockIdx.x % pairs, p = blockIdx.x / pairs;
  const int s = pair / P.Hkv, kvh = pair % P.Hkv;
  Range r;
  const int what = work_range(P, s, p, r);
  if (what == 0) return;
  if (what == 2) {
    write_zeros<__bf16, D>(P, s, kvh, lane, w);
    return;
  }

  // B operand of the QK MFMA: lane holds q[head g][kk*32 + 8*grp .. +8].
  bf16x8 qv[KK];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(P.q) + ((int64_t)s * P.H + kvh * P.G + g) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (g < P.G) x = ld16(qrow + kk * 32 + grp * 8);
      qv[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int64_t head_elems = (int64_t)kBS * D;              // one (block, kv head)
  const int64_t block_elems = head_elems * P.Hkv;           // one physical block
  const __bf16* kbase = reinterpret_cast<const __bf16*>(P.k) + kvh * head_elems;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(P.v) + kvh * head_elems;
  const int32_t* bt_row = P.bt + (int64_t)s * P.MB;

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int ntiles = (r.blk_end - r.blk_begin + TB - 1) / TB;
  for (int t = w; t < ntiles; t += NW) {
    const int b0 = r.blk_begin + t * TB;
    u32x4 kr[TB][KK];
    u32x4 vr[TB][4][NH];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      if (b0 + b < r.blk_end) {
        const int64_t phys = physical_block<TRACE>(P, bt_row, s, b0 + b, lane);
        const __bf16* kb = kbase + phys * block_elems;
        const __bf16* vb = vbase + phys * block_elems;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kr[b][kk] = ld16(kb + g * D + kk * 32 + grp * 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int h = 0; h < NH; ++h) vr[b][rr][h] = ld16(vb + (4 * grp + rr) * D + h * 128 + 8 * g);
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) kr[b][kk] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int h = 0; h < NH; ++h) vr[b][rr][h] = (u32x4){0u, 0u, 0u, 0u};
      }
    }

    // S[tok][g] for the TB blocks: lane holds tokens 4*grp + i of head g.
    f32x4 sc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      sc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        sc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[b][kk]), qv[kk],
                                                        sc[b], 0, 0, 0);
    }

    const int tok0 = b0 * kBS;
    const bool ragged = tok0 + TB * kBS > r.tok_end;  // wave-uniform
    float x[TB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float z = sc[b][i] * P.scale2;
        if (ragged && tok0 + b * kBS + 4 * grp + i >= r.tok_end) z = -INFINITY;
        x[b][i] = z;
        mx = fmaxf(mx, z);
      }
    mx = group_max(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;

    // P rounded to bf16; the exp-sum uses the same rounded values.
    __bf16 pb[TB][4];
    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[b][i] = (__bf16)fast_exp2(x[b][i] - mnew);
        ps += (float)pb[b][i];
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] *= alpha;

    // Zero V rows past the context: 0 * NaN would otherwise poison the sum.
    if (ragged) {
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (tok0 + b * kBS + 4 * grp + rr >= r.tok_end)
#pragma unroll
            for (int h = 0; h < NH; ++h) vr[b][rr][h] = (u32x4){0u, 0u, 0u, 0u};
    }

    if constexpr (TB == 2) {
      bf16x8 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = pb[0][i];
        pv[4 + i] = pb[1][i];
      }
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = j >> 1;
          u32x4 a;
          if (j & 1) {
            a[0] = pack_hi(vr[0][0][h][c], vr[0][1][h][c]);
            a[1] = pack_hi(vr[0][2][h][c], vr[0][3][h][c]);
            a[2] = pack_hi(vr[1][0][h][c], vr[1][1][h][c]);
            a[3] = pack_hi(vr[1][2][h][c], vr[1][3][h][c]);
          } else {
            a[0] = pack_lo(vr[0][0][h][c], vr[0][1][h][c]);
            a[1] = pack_lo(vr[0][2][h][c], vr[0][3][h][c]);
            a[2] = pack_lo(vr[1][0][h][c], vr[1][1][h][c]);
            a[3] = pack_lo(vr[1][2][h][c], vr[1][3][h][c]);
          }
          acc[h * 8 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pv,
                                                                   acc[h * 8 + j], 0, 0, 0);
        }
    } else {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 pv4;
#pragma unroll
      for (int i = 0; i < 4; ++i) pv4[i] = pb[0][i];
      const i16x4 pvi = __builtin_bit_cast(i16x4, pv4);
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = j >> 1;
          u32x2 a;
          if (j & 1) {
            a[0] = pack_hi(vr[0][0][h][c], vr[0][1][h][c]);
            a[1] = pack_hi(vr[0][2][h][c], vr[0][3][h][c]);
          } else {
            a[0] = pack_lo(vr[0][0][h][c], vr[0][1][h][c]);
            a[1] = pack_lo(vr[0][2][h][c], vr[0][3][h][c]);
          }
          acc[h * 8 + j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), pvi,
                                                                     acc[h * 8 + j], 0, 0, 0);
        }
    }
  }

  lsum = group_sum(lsum);
  merge_waves<NACC, NW>(acc, m, lsum, w, lane, P.G, smem);
  if (w != 0) return;
  // acc[h*8 + j][i] holds dim 128h + 32*grp + 8i + j. Reorder so that groups of
  // 4 consecutive `a` hold 4 consecutive dims: a' = h*8 + j with j%4 varying
  // fastest already does, for fixed (h, i, j/4).
  write_result<__bf16, D, NACC>(P, r, s, kvh, p, lane, acc, m, lsum, [&](int a, int i) {
    const int h = a >> 3, j = a & 7;
    return 128 * h + 32 * grp + 8 * i + j;
  });
}

// ---------------------------------------------------------------- f32 path
// 16x16x4 fp32 MFMAs: exact fp32 products, one block per tile.
template <int D, int NW, bool TRACE>
__global__ __launch_bounds__(NW * 64) void pa_partition_f32(Params P) {
  extern __shared__ float smem[];
  constexpr int NC = D / 16;    // 16-byte K loads per lane per block (4 dims each)
  constexpr int NHH = D / 64;   // 64-dim column groups of V
  constexpr int NACC = NHH * 4; // output tiles: (hh, e) -> dims 64hh + 4m + e
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15, grp = lane >> 4;

  const int pairs = P.S * P.Hkv;
  const int pair = blockIdx.x % pairs, p = blockIdx.x / pairs;
  const int s = pair / P.Hkv, kvh = pair % P.Hkv;
  Range r;
  const int what = work_range(P, s, p, r);
  if (what == 0) return;
  if (what == 2) {
    write_zeros<float, D>(P, s, kvh, lane, w);
    return;
  }

  // B operand of MFMA (c, e): q[head g][16c + 4*grp + e].
  f32x4 qv[NC];
  {
    const float* qrow = reinterpret_cast<const float*>(P.q) + ((int64_t)s * P.H + kvh * P.G + g) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (g < P.G) x = *reinterpret_cast<const f32x4*>(qrow + 16 * c + 4 * grp);
      qv[c] = x;
    }
  }

  const int64_t head_elems = (int64_t)kBS * D;
  const int64_t block_elems = head_elems * P.Hkv;
  const float* kbase = reinterpret_cast<const float*>(P.k) + kvh * head_elems;
  const float* vbase = reinterpret_cast<const float*>(P.v) + kvh * head_elems;
  const int32_t* bt_row = P.bt + (int64_t)s * P.MB;

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int nblk = r.blk_end - r.blk_begin;
  for (int t = w; t < nblk; t += NW) {
    const int blk = r.blk_begin + t;
    const int64_t phys = physical_block<TRACE>(P, bt_row, s, blk, lane);
    const float* kb = kbase + phys * block_elems;
    const float* vb = vbase + phys * block_elems;
    f32x4 kr[NC], vr[4][NHH];
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = *reinterpret_cast<const f32x4*>(kb + g * D + 16 * c + 4 * grp);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int hh = 0; hh < NHH; ++hh)
        vr[rr][hh] = *reinterpret_cast<const f32x4*>(vb + (4 * grp + rr) * D + 64 * hh + 4 * g);

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[c][e], qv[c][e], sc, 0, 0, 0);

    const int tok0 = blk * kBS;
    const bool ragged = tok0 + kBS > r.tok_end;
    float x[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float z = sc[i] * P.scale2;
      if (ragged && tok0 + 4 * grp + i >= r.tok_end) z = -INFINITY;
      x[i] = z;
      mx = fmaxf(mx, z);
    }
    mx = group_max(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    float pr[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = fast_exp2(x[i] - mnew);
      ps += pr[i];
    }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] *= alpha;
    if (ragged) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (tok0 + 4 * grp + rr >= r.tok_end)
#pragma unroll
          for (int hh = 0; hh < NHH; ++hh) vr[rr][hh] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    // MFMA (rr, hh, e): A[m][k] = V[4k + rr][64hh + 4m + e] with k = lane group.
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int hh = 0; hh < NHH; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[hh * 4 + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[rr][hh][e], pr[rr], acc[hh * 4 + e], 0, 0, 0);
  }

  lsum = group_sum(lsum);
  merge_waves<NACC, NW>(acc, m, lsum, w, lane, P.G, smem);
  if (w != 0) return;
  // acc[hh*4 + e][i] holds dim 64hh + 4*(4*grp + i) + e.
  write_result<float, D, NACC>(P, r, s, kvh, p, lane, acc, m, lsum, [&](int a, int i) {
    const int hh = a >> 2, e = a & 3;
    return 64 * hh + 16 * grp + 4 * i + e;
  });
}

// ---------------------------------------------------------------- reduce
// Phase 2: one workgroup per (sequence, head, 32-dim chunk). Thread t owns the
// float4 (t % 8) of the chunk and partitions p = t/8 (mod 32) of each group of
// 256 partitions, all loaded at once. Fixed summation order throughout.
struct ReduceParams {
  void* out;
  const float* exp_sums;
  const float* max_logits;
  const float* tmp_out;
  const int32_t* sl;
  int S, H, MB, Pmax, mode, D;
};

template <typename T>
__global__ __launch_bounds__(kReduceThreads) void pa_lse_reduce_kernel(ReduceParams R) {
  __shared__ float red[kReduceThreads / 64];
  __shared__ float cbuf[kReduceThreads];
  __shared__ f32x4 part[kReduceThreads];
  const int nchunk = R.D / kReduceChunk;
  const int dc = blockIdx.x % nchunk;
  const int sh = blockIdx.x / nchunk;
  const int s = sh / R.H;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int L = R.sl[s];
  if (L > R.MB * kBS) L = R.MB * kBS;
  if (L < 0) L = 0;
  if (R.mode == PA_MODE_AUTO && L <= kThresh) return;
  const int np = (L + kPart - 1) / kPart;
  const float* ml = R.max_logits + (int64_t)sh * R.Pmax;
  const float* es = R.exp_sums + (int64_t)sh * R.Pmax;
  const float* to = R.tmp_out + (int64_t)sh * R.Pmax * R.D + dc * kReduceChunk;

  // global max over partitions
  float mx = -INFINITY;
  for (int p = t; p < np; p += kReduceThreads) mx = fmaxf(mx, ml[p]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < kReduceThreads / 64; ++i) M = fmaxf(M, red[i]);
  __syncthreads();

  const int f4 = t & 7, pg = t >> 3;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ctot = 0.f;
  for (int base = 0; base < np; base += kReduceThreads) {
    const int p = base + t;
    const float c = (p < np) ? fast_exp2((ml[p] - M) * kLog2e) * es[p] : 0.f;
    cbuf[t] = c;
    ctot += c;
    __syncthreads();
    const int n = min(kReduceThreads, np - base);
    f32x4 v[8];
    float cw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int qq = pg + 32 * u;
      if (qq < n) {
        v[u] = *reinterpret_cast<const f32x4*>(to + (int64_t)(base + qq) * R.D + 4 * f4);
        cw[u] = cbuf[qq];
      } else {
        v[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
        cw[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += cw[u] * v[u];
    __syncthreads();
  }
  // total weight (fixed order: lanes by xor tree, then waves in order)
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ctot += __shfl_xor(ctot, o);
  if (lane == 0) red[wv] = ctot;
  part[t] = acc;
  __syncthreads();
  if (t < 8) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kReduceThreads / 64; ++i) tot += red[i];
    f32x4 sum = part[t];
    for (int g2 = 1; g2 < 32; ++g2) sum += part[g2 * 8 + t];
    const float inv = (tot > 0.f) ? 1.f / tot : 0.f;
    T* row = reinterpret_cast<T*>(R.out) + (int64_t)sh * R.D + dc * kReduceChunk;
    store4<T>(row, 4 * t, sum * inv);
  }
}

// ---------------------------------------------------------------- host side
constexpr int kNW = 4;  // waves per partition workgroup

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(const pa_shape* sh) {
  if (!sh) return PA_EINVAL;
  if (sh->num_seqs < 0 || sh->num_heads < 1 || sh->num_kv_heads < 1 || sh->max_blocks_per_seq < 1 ||
      sh->num_blocks < 1)
    return PA_EINVAL;
  if (sh->num_heads % sh->num_kv_heads != 0) return PA_EINVAL;
  if (sh->num_heads / sh->num_kv_heads > 16) return PA_EUNSUPPORTED;
  if (sh->head_dim != 128 && sh->head_dim != 256) return PA_EUNSUPPORTED;
  if (sh->block_size != kBS) return PA_EUNSUPPORTED;
  if (sh->dtype != PA_F32 && sh->dtype != PA_BF16) return PA_EUNSUPPORTED;
  if (sh->max_blocks_per_seq > (1 << 26)) return PA_EUNSUPPORTED;  // keeps token counts in int32
  return PA_OK;
}

int64_t max_partitions(const pa_shape* sh) {
  return ((int64_t)sh->max_blocks_per_seq * kBS + kPart - 1) / kPart;
}

int check_all(const void* out, const void* q, const void* k, const void* v, const int32_t* bt,
              const int32_t* sl, const pa_shape* sh, const float* es, const float* ml,
              const float* to, int mode, bool need_partials, bool need_inputs) {
  const int st = check_shape(sh);
  if (st != PA_OK) return st;
  if (mode != PA_MODE_AUTO && mode != PA_MODE_V1 && mode != PA_MODE_V2) return PA_EUNSUPPORTED;
  if (sh->num_seqs == 0) return PA_OK;  // empty batch: nothing is read or written
  if (!out || !sl) return PA_EINVAL;
  if (need_inputs && (!q || !k || !v || !bt)) return PA_EINVAL;
  if (need_partials && (!es || !ml || !to)) return PA_EINVAL;
  if (!aligned(out, 16) || !aligned(sl, 4)) return PA_EALIGN;
  if (need_inputs && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(bt, 4)))
    return PA_EALIGN;
  if (need_partials && (!aligned(es, 4) || !aligned(ml, 4) || !aligned(to, 16))) return PA_EALIGN;
  // grid size and 32-bit thread ids
  const int64_t pgrid = (mode == PA_MODE_V1) ? 1 : max_partitions(sh);
  const int64_t wgs = (int64_t)sh->num_seqs * sh->num_kv_heads * pgrid;
  if (wgs * kNW * 64 >= (int64_t)1 << 31) return PA_EUNSUPPORTED;
  if ((int64_t)sh->num_seqs * sh->num_heads * (sh->head_dim / kReduceChunk) * kReduceThreads >= (int64_t)1 << 31)
    return PA_EUNSUPPORTED;
  return PA_OK;
}

template <int NACC>
size_t partition_smem(int G) {
  return (size_t)2 * kNW * 16 * sizeof(float) + (size_t)(kNW - 1) * NACC * G * 4 * sizeof(f32x4);
}

hipError_t launch_partitions(const Params& P, int D, int dtype, bool trace, hipStream_t stream) {
  const int64_t pgrid = (P.mode == PA_MODE_V1) ? 1 : P.Pmax;
  const dim3 grid((unsigned)((int64_t)P.S * P.Hkv * pgrid));
  const dim3 block(kNW * 64);
  if (grid.x == 0) return hipSuccess;
  if (dtype == PA_BF16) {
    if (D == 128) {
      auto kern = trace ? pa_partition_bf16<128, kNW, 2, true> : pa_partition_bf16<128, kNW, 2, false>;
      hipLaunchKernelGGL(kern, grid, block, partition_smem<8>(P.G), stream, P);
    } else {
      auto kern = trace ? pa_partition_bf16<256, kNW, 1, true> : pa_partition_bf16<256, kNW, 1, false>;
      hipLaunchKernelGGL(kern, grid, block, partition_smem<16>(P.G), stream, P);
    }
  } else {
    if (D == 128) {
      auto kern = trace ? pa_partition_f32<128, kNW, true> : pa_partition_f32<128, kNW, false>;
      hipLaunchKernelGGL(kern, grid, block, partition_smem<8>(P.G), stream, P);
    } else {
      auto kern = trace ? pa_partition_f32<256, kNW, true> : pa_partition_f32<256, kNW, false>;
      hipLaunchKernelGGL(kern, grid, block, partition_smem<16>(P.G), stream, P);
    }
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& R, int dtype, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)R.S * R.H * (R.D / kReduceChunk)));
  if (grid.x == 0) return hipSuccess;
  if (dtype == PA_BF16)
    hipLaunchKernelGGL(pa_lse_reduce_kernel<__bf16>, grid, dim3(kReduceThreads), 0, stream, R);
  else
    hipLaunchKernelGGL(pa_lse_reduce_kernel<float>, grid, dim3(kReduceThreads), 0, stream, R);
  return hipGetLastError();
}

Params make_params(void* out, const void* q, const void* k, const void* v, const int32_t* bt,
                   const int32_t* sl, const pa_shape* sh, float scale, float* es, float* ml,
                   float* to, int mode, int32_t* trace, int32_t* err) {
  Params P;
  P.q = q; P.k = k; P.v = v; P.bt = bt; P.sl = sl; P.out = out;
  P.exp_sums = es; P.max_logits = ml; P.tmp_out = to; P.trace = trace; P.err = err;
  P.NB = sh->num_blocks;
  P.S = sh->num_seqs; P.H = sh->num_heads; P.Hkv = sh->num_kv_heads;
  P.G = sh->num_heads / sh->num_kv_heads; P.MB = sh->max_blocks_per_seq;
  P.Pmax = (int)max_partitions(sh); P.mode = mode;
  P.scale2 = scale * kLog2e;
  return P;
}

ReduceParams make_reduce_params(void* out, const float* es, const float* ml, const float* to,
                                const int32_t* sl, const pa_shape* sh, int mode) {
  ReduceParams R;
  R.out = out; R.exp_sums = es; R.max_logits = ml; R.tmp_out = to; R.sl = sl;
  R.S = sh->num_seqs; R.H = sh->num_heads; R.MB = sh->max_blocks_per_seq;
  R.Pmax = (int)max_partitions(sh); R.mode = mode; R.D = sh->head_dim;
  return R;
}

int run_partitions(void* out, const void* q, const void* k, const void* v, const int32_t* bt,
                   const int32_t* sl, const pa_shape* sh, float scale, float* es, float* ml,
                   float* to, int mode, int32_t* trace, int32_t* err, void* stream) {
  const int st = check_all(out, q, k, v, bt, sl, sh, es, ml, to, mode, mode != PA_MODE_V1, true);
  if (st != PA_OK) return st;
  (void)hipGetLastError();
  const Params P = make_params(out, q, k, v, bt, sl, sh, scale, es, ml, to, mode, trace, err);
  if (launch_partitions(P, sh->head_dim, sh->dtype, trace != nullptr || err != nullptr,
                        (hipStream_t)stream) != hipSuccess)
    return PA_EHIP;
  return PA_OK;
}

int run_reduce(void* out, const float* es, const float* ml, const float* to, const int32_t* sl,
               const pa_shape* sh, int mode, void* stream) {
  const int st = check_all(out, nullptr, nullptr, nullptr, nullptr, sl, sh, es, ml, to, mode, true, false);
  if (st != PA_OK) return st;
  if (mode == PA_MODE_V1) return PA_OK;  // nothing is partitioned
  (void)hipGetLastError();
  const ReduceParams R = make_reduce_params(out, es, ml, to, sl, sh, mode);
  if (launch_reduce(R, sh->dtype, (hipStream_t)stream) != hipSuccess) return PA_EHIP;
  return PA_OK;
}

int run_full(void* out, const void* q, const void* k, const void* v, const int32_t* bt,
             const int32_t* sl, const pa_shape* sh, float scale, float* es, float* ml, float* to,
             int mode, void* stream) {
  const int st = check_all(out, q, k, v, bt, sl, sh, es, ml, to, mode, mode != PA_MODE_V1, true);
  if (st != PA_OK) return st;
  int rc = run_partitions(out, q, k, v, bt, sl, sh, scale, es, ml, to, mode, nullptr, nullptr, stream);
  if (rc != PA_OK || mode == PA_MODE_V1) return rc;
  return run_reduce(out, es, ml, to, sl, sh, mode, stream);
}

}  // namespace

extern "C" {

int pa_decode_v1(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                 float scale, void* stream) {
  return run_full(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, nullptr, nullptr,
                  nullptr, PA_MODE_V1, stream);
}

int pa_decode_v2(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                 float scale, float* exp_sums, float* max_logits, float* tmp_out, void* stream) {
  return run_full(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, exp_sums,
                  max_logits, tmp_out, PA_MODE_V2, stream);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
              float scale, float* exp_sums, float* max_logits, float* tmp_out, void* stream) {
  return run_full(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, exp_sums,
                  max_logits, tmp_out, PA_MODE_AUTO, stream);
}

int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const pa_shape* shape, float scale, float* exp_sums, float* max_logits,
                         float* tmp_out, int mode, void* stream) {
  return run_partitions(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, exp_sums,
                        max_logits, tmp_out, mode, nullptr, nullptr, stream);
}

int pa_lse_reduce(void* out, const float* exp_sums, const float* max_logits, const float* tmp_out,
                  const int32_t* seq_lens, const pa_shape* shape, int mode, void* stream) {
  return run_reduce(out, exp_sums, max_logits, tmp_out, seq_lens, shape, mode, stream);
}

int pa_decode_partitions_debug(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               const pa_shape* shape, float scale, float* exp_sums,
                               float* max_logits, float* tmp_out, int mode,
                               int32_t* gather_trace, int32_t* err_flag, void* stream) {
  if (gather_trace && !aligned(gather_trace, 4)) return PA_EALIGN;
  if (err_flag && !aligned(err_flag, 4)) return PA_EALIGN;
  return run_partitions(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, exp_sums,
                        max_logits, tmp_out, mode, gather_trace, err_flag, stream);
}

int64_t pa_max_partitions(const pa_shape* shape) {
  const int st = check_shape(shape);
  if (st != PA_OK) return st;
  return max_partitions(shape);
}

int64_t pa_partials_elems(const pa_shape* shape, int which) {
  const int st = check_shape(shape);
  if (st != PA_OK) return st;
  const int64_t n = (int64_t)shape->num_seqs * shape->num_heads * max_partitions(shape);
  if (which == 0) return n;
  if (which == 1) return n * shape->head_dim;
  return PA_EINVAL;
}

int pa_check_args(const void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                  const float* exp_sums, const float* max_logits, const float* tmp_out, int mode) {
  return check_all(out, q, k_cache, v_cache, block_tables, seq_lens, shape, exp_sums, max_logits,
                   tmp_out, mode, mode != PA_MODE_V1, true);
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument (null pointer, bad size, or num_heads % num_kv_heads != 0)";
    case PA_EUNSUPPORTED: return "unsupported configuration (head_dim, block_size, group size, dtype, mode or size)";
    case PA_EALIGN: return "pointer not aligned (16 bytes for q/caches/out/tmp_out, 4 for int32/f32 arrays)";
    case PA_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int pa_version(void) { return 1; }

}  // extern "C"
