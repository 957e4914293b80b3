// Paged-attention decode for gfx950 (MI355X): HIP kernels and the C ABI.
//
// Method (project_6 commit cd0d9e1a, qwen3_6_scripts):
//   * "paged_attn.py rewrite", item 2: a sequence whose context is longer than
//     8192 tokens takes the partitioned path (V2), the others one pass (V1).
//   * "V2 implementation": phase 1 runs attention over each 512-token
//     partition and keeps its max logit, exp-sum and output; phase 2 combines
//     partitions with log-sum-exp weights. Inside a partition the softmax is
//     the running (online) form, the same blocking flash attention uses.
//   * Partition size: 512 tokens. The prefix-prefill patch docstring (project_6
//     blame of optimizations/prefix_prefill_patch.py) records 256 as the other
//     size once in use; a shape may opt into it (pa_shape.partition_size).
//
// Kernel design (gfx950, wave64):
//   One workgroup per work item: (sequence, KV head) for a single pass,
//   (sequence, KV head, partition) otherwise. Batches map workgroups through
//   a compact work list built from seq_lens on the device (item_of), with the
//   long single-pass items first and the unused workgroups at the end. Each
//   wave walks "tiles" of whole 16-token blocks, several in flight at a time
//   where the launch shape asks for it. For a tile it
//     - loads K as whole rows and transposes it through a swizzled LDS tile
//       so that lane (tok = l%16, grp = l/16) holds 8 consecutive head dims
//       of token tok: the A operand of a 16x16x32 bf16 MFMA whose M axis is
//       the 16 tokens and whose N axis is the GQA group (padded to 16), so
//       one load of K serves every query head of the group;
//     - computes S[tok][g] = K q^T, leaving lane l with 4 tokens of head l%16;
//     - keeps a running max / exp-sum per head (two xor-shuffles per tile);
//     - computes O^T[d][g] += V^T[d][tok] P[tok][g]: the B operand P is the QK
//       accumulator itself (rounded to bf16), and V is loaded as whole rows
//       (16 lanes x 16 B = one 256-byte row) and transposed in registers.
//   Waves then merge (max, exp-sum, output) through LDS in a fixed order and
//   the workgroup writes either out (V1) or the three partials (V2).
//
// Data errors never turn into out-of-bounds accesses: contexts are cut to the
// table width and out-of-range block ids are read as block 0 (both reported
// through the optional error word).

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "pa_common.h"

namespace {

constexpr int kPart = PA_PARTITION_SIZE;
constexpr int kThresh = PA_V2_THRESHOLD;
constexpr int kReduceThreads = 256;
constexpr int kReduceChunk = 32;   // head dims per reduce workgroup
constexpr int kCompactMaxSeqs = 1024;  // largest batch mapped through the compact work list

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
  int PS;        // tokens per partition (512, or the opt-in 256)
  int compact;   // workgroups follow the compact work list (item_of)
  float scale2;  // softmax scale times log2(e): logits are kept in base-2 units
};

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
    const int np = (L + P.PS - 1) / P.PS;
    if (p >= np) return 0;
    r.tok_begin = p * P.PS;
    r.tok_end = min(r.tok_begin + P.PS, L);
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

// Work item of workgroup b in the compact order, computed by every wave from
// seq_lens alone: first one item per KV head for every sequence that takes a
// single pass (a zero-length context included: it writes zeros), in sequence
// order; then, sequence by sequence, the partitions of every partitioned
// sequence as (partition, KV head) pairs. Workgroups past the last item
// return false. The host sizes the grid for the widest table, so the unused
// workgroups trail the used ones instead of sitting between them (a read of
// the 512-token items of 64 mixed-length sequences took 219 us among
// interleaved empty workgroups and 164 us compact), and the long single-pass
// items go first so that they do not finish last.
//
// clamp_len: sequence s's length as the kernels use it (cut to the table's
// width, negative lengths read as zero); work_range reports the cut.
__device__ __forceinline__ int clamp_len(const Params& P, int s) {
  int L = P.sl[s];
  const int cap = P.MB * kBS;
  L = L > cap ? cap : L;
  return L < 0 ? 0 : L;
}

// item_of: the work item of workgroup b in the compact order described above.
__device__ __forceinline__ bool item_of(const Params& P, int b, int lane, int& s_out, int& kvh_out,
                                        int& p_out) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes < this one
  // Pass 1, in every workgroup: the number of single-pass sequences (AUTO
  // mode only) and of partitions. The lengths of eight 64-sequence chunks are
  // loaded into registers before any of them is used, so their loads are in
  // flight together. Workgroups past the last item leave after this pass.
  constexpr int kLenChunks = 8;
  int n1 = 0, np = 0;
  for (int c0 = 0; c0 < P.S; c0 += kLenChunks * 64) {
    int len[kLenChunks];
#pragma unroll
    for (int u = 0; u < kLenChunks; ++u)  // unconditional loads (index clamped into the batch)
      len[u] = P.sl[min(c0 + 64 * u + lane, P.S - 1)];
#pragma unroll
    for (int u = 0; u < kLenChunks; ++u) {
      const int L = len[u] > P.MB * kBS ? P.MB * kBS : len[u];
      len[u] = (c0 + 64 * u + lane < P.S) ? (L < 0 ? 0 : L) : -1;
    }
#pragma unroll
    for (int u = 0; u < kLenChunks; ++u) {
      const bool one = len[u] >= 0 && P.mode == PA_MODE_AUTO && len[u] <= kThresh;
      n1 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(one));
      if (len[u] >= 0 && !one) np += (len[u] + P.PS - 1) / P.PS;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) np += __shfl_xor(np, o);
  const int total1 = n1 * P.Hkv;
  if (b >= total1 + np * P.Hkv) return false;
  if (b < total1) {
    int r = b / P.Hkv;  // rank of the sequence among the single-pass ones
    for (int c = 0; c < P.S; c += 64) {
      const int s = c + lane;
      const bool one = s < P.S && clamp_len(P, s) <= kThresh;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(one);
      const int cnt = __builtin_popcountll(mask);
      if (r < cnt) {
        const bool hit = one && __builtin_popcountll(mask & below) == r;
        s_out = __builtin_amdgcn_readfirstlane(c + __builtin_ctzll(__builtin_amdgcn_ballot_w64(hit)));
        kvh_out = b % P.Hkv;
        p_out = 0;
        return true;
      }
      r -= cnt;
    }
    return false;
  }
  // Pass 2: partitioned sequences, Hkv * ceil(L / PS) items each.
  int r = b - total1;
  for (int c = 0; c < P.S; c += 64) {
    const int s = c + lane;
    int n = 0;
    if (s < P.S) {
      const int L = clamp_len(P, s);
      if (P.mode == PA_MODE_V2 || L > kThresh) n = (L + P.PS - 1) / P.PS * P.Hkv;
    }
    int incl = n;  // inclusive prefix sum over the chunk's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int tot = __shfl(incl, 63);
    if (r < tot) {
      const bool hit = n > 0 && r >= incl - n && r < incl;
      const int l = __builtin_ctzll(__builtin_amdgcn_ballot_w64(hit));
      const int local = __builtin_amdgcn_readfirstlane(r - (__shfl(incl, l) - __shfl(n, l)));
      s_out = c + l;
      p_out = local / P.Hkv;
      kvh_out = local % P.Hkv;
      return true;
    }
    r -= tot;
  }
  return false;
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

// Store of 4 floats of a V2 partial row, write-through at system scope (sc1):
// on the largest batch these rows cost ~20% less than with plain stores,
// where they trickle out of the L2 between the K/V reads.
__device__ __forceinline__ void store4_partial(float* row, int d, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(row + d), "v"(v) : "memory");
}

// Merge the per-wave (max, exp-sum, output) triples of one workgroup and
// write the result. acc holds the wave's unnormalised output for head
// g = lane%16 relative to its running max m (base 2), lsum its exp-sum;
// dim_of(a, i) names the head dim held in acc[a][i] (dims a..a+3 of one i are
// consecutive for a multiple of 4).
//
// Every wave stores its (max, exp-sum) and its unscaled output rows in its
// own LDS area ([wave][head][D] rows, apart from the main loop's scratch, so
// no wave waits for another before writing); after one barrier all threads
// rescale and sum the waves in a fixed order (bitwise deterministic) and
// write whole output rows with consecutive 16-byte stores, so every row goes
// out as full cache lines: rows written in scattered 16-byte pieces measured
// about 15% slower on the largest batch.
template <typename T, int D, int NACC, int NW, typename DimOf>
__device__ __forceinline__ void merge_and_write(const Params& P, const Range& r, int s, int kvh,
                                                int p, int w, int lane, const f32x4 (&acc)[NACC],
                                                float m, float lsum, float* smem, DimOf dim_of) {
  constexpr int RS = D + 4;  // padded LDS row (floats): rows of different heads hit different banks
  const int G = P.G;
  const int g = lane & 15;
  float* sm_m = smem;
  float* sm_l = smem + NW * 16;
  float* sm_o = smem + 2 * NW * 16;
  if (lane < 16) {
    sm_m[w * 16 + g] = m;
    sm_l[w * 16 + g] = lsum;
  }
  if (g < G) {
    float* row = sm_o + ((size_t)w * G + g) * RS;
#pragma unroll
    for (int a = 0; a < NACC; a += 4)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(row + dim_of(a, i)) = (f32x4){acc[a][i], acc[a + 1][i], acc[a + 2][i], acc[a + 3][i]};
  }
  __syncthreads();
  const int t = threadIdx.x;
  for (int e = t * 4; e < G * D; e += NW * 64 * 4) {
    const int hg = e / D, d = e % D;
    float Mg = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) Mg = fmaxf(Mg, sm_m[i * 16 + hg]);
    float lt = 0.f;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const float mi = sm_m[i * 16 + hg];
      const float f = (mi > -INFINITY) ? fast_exp2(mi - Mg) : 0.f;
      lt += sm_l[i * 16 + hg] * f;
      sum += f * *reinterpret_cast<const f32x4*>(sm_o + ((size_t)i * G + hg) * RS + d);
    }
    const float inv = 1.f / lt;
    const int64_t sh = (int64_t)s * P.H + kvh * G + hg;
    if (!r.v2) {
      store4<T>(reinterpret_cast<T*>(P.out) + sh * D, d, sum * inv);
    } else {
      store4_partial(P.tmp_out + (sh * P.Pmax + p) * D, d, sum * inv);
      if (d == 0) {
        P.exp_sums[sh * P.Pmax + p] = lt;
        P.max_logits[sh * P.Pmax + p] = Mg * kLn2;  // back to natural-log units
      }
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void write_zeros(const Params& P, int s, int kvh, int nthreads) {
  T* rows = reinterpret_cast<T*>(P.out) + ((int64_t)s * P.H + kvh * P.G) * D;  // G consecutive rows
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int e = threadIdx.x * 4; e < P.G * D; e += nthreads * 4) store4<T>(rows, e, z);
}

// ---------------------------------------------------------------- 16-bit path
// Per wave, tiles of TB whole blocks are streamed through a ring of NBUF
// register tiles (the launch shapes set TB and NBUF), in straight-line
// chunks whose loads carry no branch (see the tile loop in the kernel).
//
// Loads: both K and V are read as whole rows: lane (g = l%16, grp = l/16)
// reads 16 bytes at row 4*grp + rr, dims 128h + 8g .. +8, so 16 consecutive
// lanes cover one 256-byte row segment (coalesced). V is transposed in
// registers for the P.V MFMA. K must reach the QK MFMA with one token per
// lane%16, so it takes a round trip through a wave-private LDS tile whose
// 16-byte chunks are XOR-swizzled by row: both the row-wise writes and the
// token-wise MFMA reads then touch 16 distinct bank groups.
//
// Block ids: each wave keeps the physical ids of its next 64 blocks in one
// VGPR (lane j holds one id) and reads them with readlane, so no tile waits on
// a table load of its own.

// Per-wave list of physical block ids: lane j holds the id of block (j % TB)
// of the wave's tile t0 + (first_k + j / TB) * dt, for tiles starting at
// blk_begin. The table read itself needs only the partition index, so the
// first list is read before seq_lens is known (entries past the table width
// are skipped); check_block_ids() then applies the context length.
template <int TB>
__device__ __forceinline__ int read_block_ids(const Params& P, const int32_t* bt_row, int blk_begin,
                                              int t0, int dt, int first_k, int lane) {
  const int k = first_k + lane / TB;
  const int blk = blk_begin + (t0 + k * dt) * TB + lane % TB;
  return blk < P.MB ? bt_row[blk] : -1;
}

template <bool TRACE, int TB>
__device__ __forceinline__ int check_block_ids(const Params& P, int id, int s, const Range& r, int t0,
                                               int dt, int first_k, int lane) {
  const int k = first_k + lane / TB;
  const int blk = r.blk_begin + (t0 + k * dt) * TB + lane % TB;
  if (blk >= r.blk_end) return -1;
  if ((uint64_t)(int64_t)id >= (uint64_t)P.NB) {
    if (P.err) atomicOr(P.err, 2);
    id = 0;
  }
  if (TRACE && P.trace) P.trace[(int64_t)s * P.MB + blk] = id;
  return id;
}

// NBUF: tiles of the wave in flight at once. Each wave keeps a ring of NBUF
// register tiles: the loads of tiles k+1 .. k+NBUF-1 are outstanding while
// tile k is computed, and tile k's buffer takes the loads of tile k+NBUF as
// soon as its math is done. WPE: the waves per SIMD the register allocation
// must allow (a deeper ring needs fewer, larger waves).
template <typename T, int D, int NW, int TB, int NBUF, int CT, int WPE, bool TRACE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void pa_partition_h16(Params P) {
  typedef typename H16<T>::x8 tx8;
  typedef typename H16<T>::x4 tx4;
  extern __shared__ float smem[];
  constexpr int KK = D / 32;    // QK MFMAs per block (32 dims each)
  constexpr int NH = D / 128;   // 128-dim column groups
  constexpr int NACC = NH * 8;  // output tiles: (h, j) -> dims 128h + 8m + j
  constexpr int CH = 64 / TB;   // tiles per block-id refill
  constexpr int KCH = D / 8;    // 16-byte chunks per K row
  static_assert(NBUF >= 1 && NBUF <= CT && CH % CT == 0, "ring depth and chunk size");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15, grp = lane >> 4;

  // Workgroup b serves (pair b % pairs, partition b / pairs): its NW waves
  // take the item's tiles t0, t0 + dt, ... and merge through LDS at the end.
  // (compact grids map workgroups through item_of instead).
  const int pairs = P.S * P.Hkv;
  int pair = blockIdx.x % pairs, p = blockIdx.x / pairs;
  const int t0 = w, dt = NW;
  int s = pair / P.Hkv, kvh = pair % P.Hkv;
  if (P.compact && !item_of(P, blockIdx.x, lane, s, kvh, p)) return;
  const int32_t* bt_row = P.bt + (int64_t)s * P.MB;
  // The first block-id list, read speculatively (a single pass starts at block
  // 0, partition p at block 32p; a workgroup with nothing to do drops it).
  int ids = read_block_ids<TB>(P, bt_row, (P.mode == PA_MODE_V1) ? 0 : p * (P.PS / kBS), t0, dt, 0, lane);
  Range r;
  const int what = work_range(P, s, p, r);
  if (what == 0) return;
  if (what == 2) {
    write_zeros<T, D>(P, s, kvh, NW * 64);
    return;
  }

  // LDS: [wave max | wave exp-sum][merge rows: NW x G x (D + 4) floats][per-wave K tiles].
  u32x4* ktile = reinterpret_cast<u32x4*>(smem + 2 * NW * 16 + (size_t)NW * P.G * (D + 4)) + (size_t)w * TB * 16 * KCH;

  // B operand of the QK MFMA: lane holds q[head g][kk*32 + 8*grp .. +8].
  tx8 qv[KK];
  {
    const T* qrow = reinterpret_cast<const T*>(P.q) + ((int64_t)s * P.H + kvh * P.G + g) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (g < P.G) x = ld16(qrow + kk * 32 + grp * 8);
      qv[kk] = __builtin_bit_cast(tx8, x);
    }
  }

  const int64_t head_elems = (int64_t)kBS * D;     // one (block, kv head)
  const int64_t block_elems = head_elems * P.Hkv;  // one physical block
  const T* kbase = reinterpret_cast<const T*>(P.k) + kvh * head_elems;
  const T* vbase = reinterpret_cast<const T*>(P.v) + kvh * head_elems;

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int ntiles = (r.blk_end - r.blk_begin + TB - 1) / TB;
  ids = check_block_ids<TRACE, TB>(P, ids, s, r, t0, dt, 0, lane);

  auto compute = [&](BTile<D, TB>& tl, int t) {
    // K: registers -> swizzled LDS tile -> MFMA operand layout.
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const int row = 4 * grp + rr, c16 = 16 * h + g;
          ktile[(b * 16 + row) * KCH + (c16 ^ row)] = tl.k[b][rr][h];
        }
    f32x4 sc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      sc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int c16 = 4 * kk + grp;
        const u32x4 kr = ktile[(b * 16 + g) * KCH + (c16 ^ g)];
        sc[b] = H16<T>::mma32(__builtin_bit_cast(tx8, kr), qv[kk], sc[b]);
      }
    }

    const int tok0 = (r.blk_begin + t * TB) * kBS;
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

    // P rounded to the cache's 16-bit type; the exp-sum uses the same rounded values.
    T pb[TB][4];
    float ps = 0.f;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[b][i] = (T)fast_exp2(x[b][i] - mnew);
        ps += (float)pb[b][i];
      }
    lsum = lsum * alpha + ps;
    // Rescale only when some head's running max moved (alpha == 1 otherwise).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) acc[a] *= alpha;
    }

    // Zero V rows past the context: 0 * NaN would otherwise poison the sum.
    if (ragged) {
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (tok0 + b * kBS + 4 * grp + rr >= r.tok_end)
#pragma unroll
            for (int h = 0; h < NH; ++h) tl.v[b][rr][h] = (u32x4){0u, 0u, 0u, 0u};
    }

    if constexpr (TB == 2) {
      tx8 pv;
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
            a[0] = pack_hi(tl.v[0][0][h][c], tl.v[0][1][h][c]);
            a[1] = pack_hi(tl.v[0][2][h][c], tl.v[0][3][h][c]);
            a[2] = pack_hi(tl.v[1][0][h][c], tl.v[1][1][h][c]);
            a[3] = pack_hi(tl.v[1][2][h][c], tl.v[1][3][h][c]);
          } else {
            a[0] = pack_lo(tl.v[0][0][h][c], tl.v[0][1][h][c]);
            a[1] = pack_lo(tl.v[0][2][h][c], tl.v[0][3][h][c]);
            a[2] = pack_lo(tl.v[1][0][h][c], tl.v[1][1][h][c]);
            a[3] = pack_lo(tl.v[1][2][h][c], tl.v[1][3][h][c]);
          }
          acc[h * 8 + j] = H16<T>::mma32(__builtin_bit_cast(tx8, a), pv, acc[h * 8 + j]);
        }
    } else {
      tx4 pv4;
#pragma unroll
      for (int i = 0; i < 4; ++i) pv4[i] = pb[0][i];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = j >> 1;
          u32x2 a;
          if (j & 1) {
            a[0] = pack_hi(tl.v[0][0][h][c], tl.v[0][1][h][c]);
            a[1] = pack_hi(tl.v[0][2][h][c], tl.v[0][3][h][c]);
          } else {
            a[0] = pack_lo(tl.v[0][0][h][c], tl.v[0][1][h][c]);
            a[1] = pack_lo(tl.v[0][2][h][c], tl.v[0][3][h][c]);
          }
          acc[h * 8 + j] = H16<T>::mma16(__builtin_bit_cast(tx4, a), pv4, acc[h * 8 + j]);
        }
    }
  };

  // The wave's tiles go in chunks of CT, each chunk straight-line code with
  // NB tiles in flight: tile k's buffer takes the loads of tile k + NB once
  // tile k is computed. A partition is one chunk; a long single pass takes
  // several, with the ring refilled at the start of each. Tiles past the
  // item's end load nothing (zero-length resources) and skip the math.
  const int nk = t0 < ntiles ? (ntiles - t0 + dt - 1) / dt : 0;  // this wave's tiles
  auto stream_tiles = [&](auto nb_const) {
    constexpr int NB = decltype(nb_const)::value;
    for (int k0 = 0; k0 < nk; k0 += CT) {
      auto issue = [&](BTile<D, TB>& tl, int k) {
        int64_t phys[TB];
        bool valid[TB];
        const int t = t0 + k * dt;
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          valid[b] = k < nk && r.blk_begin + t * TB + b < r.blk_end;
          phys[b] = __builtin_amdgcn_readlane(ids, (k % CH) * TB + b);
        }
        issue_tile_rsrc<T, D, TB>(tl, kbase, vbase, block_elems, phys, valid, g, grp);
      };
      if (k0 > 0 && k0 % CH == 0)
        ids = check_block_ids<TRACE, TB>(P, read_block_ids<TB>(P, bt_row, r.blk_begin, t0, dt, k0, lane), s, r,
                                         t0, dt, k0, lane);
      BTile<D, TB> ring[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) issue(ring[j], k0 + j);
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const int k = k0 + j;
        if (k < nk) compute(ring[j % NB], t0 + k * dt);
        if (j + NB < CT) issue(ring[j % NB], k + NB);
      }
    }
  };
  stream_tiles(std::integral_constant<int, NBUF>{});

  lsum = group_sum(lsum);
  // acc[h*8 + j][i] holds dim 128h + 32*grp + 8i + j.
  merge_and_write<T, D, NACC, NW>(P, r, s, kvh, p, w, lane, acc, m, lsum, smem, [&](int a, int i) {
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
  int pair = blockIdx.x % pairs, p = blockIdx.x / pairs;
  int s = pair / P.Hkv, kvh = pair % P.Hkv;
  if (P.compact && !item_of(P, blockIdx.x, lane, s, kvh, p)) return;
  Range r;
  const int what = work_range(P, s, p, r);
  if (what == 0) return;
  if (what == 2) {
    write_zeros<float, D>(P, s, kvh, NW * 64);
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
  // acc[hh*4 + e][i] holds dim 64hh + 4*(4*grp + i) + e.
  merge_and_write<float, D, NACC, NW>(P, r, s, kvh, p, w, lane, acc, m, lsum, smem, [&](int a, int i) {
    const int hh = a >> 2, e = a & 3;
    return 64 * hh + 16 * grp + 4 * i + e;
  });
}

// ---------------------------------------------------------------- reduce
// Phase 2 (project_6 commit cd0d9e1a, "V2 implementation", phase 2): one
// workgroup per (sequence, head, CW-wide slice of the head dims). Thread t
// owns float4 t % (CW/4) of the slice and partitions t / (CW/4) + PG*u of
// each group of PG*NU partitions; all loads of a group are issued at once
// and folded into the thread's running (max, weight sum, output), rescaled
// when its max grows. The threads holding the same float4 then merge their
// triples: first across the lanes of a wave (xor-shuffles), then the waves'
// results through LDS, in a fixed order (bitwise deterministic).
// The host picks CW: full rows (one coalesced 1 KB row per wave at D = 256)
// when there are enough (sequence, head) rows to fill the GPU, narrow slices
// (more workgroups) otherwise.
// With SPEC (small partial sets, where the kernel is latency-bound) the first
// group's loads go out before the sequence length arrives, bounded by Pmax,
// and entries past the sequence's partition count are masked afterwards.
struct ReduceParams {
  void* out;
  const float* exp_sums;
  const float* max_logits;
  const float* tmp_out;
  const int32_t* sl;
  int S, H, MB, Pmax, mode, D, PS;
};

// Merge (M, c, acc) with another triple of the same slice position: both are
// rescaled to the larger max (natural-log units); an empty triple has M = -inf.
__device__ __forceinline__ void merge_triple(float& M, float& c, f32x4& acc, float Mo, float co, f32x4 ao) {
  const float Mn = fmaxf(M, Mo);
  if (Mn == -INFINITY) return;
  const float fa = (M > -INFINITY) ? fast_exp2((M - Mn) * kLog2e) : 0.f;
  const float fb = (Mo > -INFINITY) ? fast_exp2((Mo - Mn) * kLog2e) : 0.f;
  acc = acc * fa + ao * fb;
  c = c * fa + co * fb;
  M = Mn;
}

template <typename T, int CW, bool SPEC>
__global__ __launch_bounds__(kReduceThreads) void pa_lse_reduce_kernel(ReduceParams R) {
  constexpr int F4 = CW / 4;                 // float4 per slice
  constexpr int PG = kReduceThreads / F4;    // partition groups
  constexpr int NU = 16;                     // partitions per thread per group
  constexpr int NWV = kReduceThreads / 64;   // waves
  static_assert(F4 <= 64 && 64 % F4 == 0, "slice width");
  __shared__ float sm_m[NWV][F4], sm_c[NWV][F4];
  __shared__ f32x4 sm_a[NWV][F4];
  const int nchunk = R.D / CW;
  const int dc = blockIdx.x % nchunk;
  const int sh = blockIdx.x / nchunk;
  const int s = sh / R.H;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const float* ml = R.max_logits + (int64_t)sh * R.Pmax;
  const float* es = R.exp_sums + (int64_t)sh * R.Pmax;
  const float* to = R.tmp_out + (int64_t)sh * R.Pmax * R.D + dc * CW;
  const int f4 = t % F4, pg = t / F4;
  float mv[NU], ev[NU];
  f32x4 v[NU];
  auto load_group = [&](int base, int limit) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int pp = base + pg + PG * u;
      if (pp < limit) {
        mv[u] = ml[pp];
        ev[u] = es[pp];
        v[u] = *reinterpret_cast<const f32x4*>(to + (int64_t)pp * R.D + 4 * f4);
      } else {
        mv[u] = -INFINITY;
        ev[u] = 0.f;
        v[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  if constexpr (SPEC) load_group(0, R.Pmax);
  int L = R.sl[s];
  if (L > R.MB * kBS) L = R.MB * kBS;
  if (L < 0) L = 0;
  if (R.mode == PA_MODE_AUTO && L <= kThresh) return;
  const int np = (L + R.PS - 1) / R.PS;

  // The thread's running (max, weight sum, weighted output) over its own
  // partitions, rescaled when its max grows.
  float M = -INFINITY, ctot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < np; base += PG * NU) {
    if (SPEC && base == 0) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (pg + PG * u >= np) {
          mv[u] = -INFINITY;
          ev[u] = 0.f;
          v[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      }
    } else {
      load_group(base, np);
    }
    float cm = mv[0];
#pragma unroll
    for (int u = 1; u < NU; ++u) cm = fmaxf(cm, mv[u]);
    const float Mn = fmaxf(M, cm);
    if (Mn > -INFINITY) {
      const float a = (M > -INFINITY) ? fast_exp2((M - Mn) * kLog2e) : 0.f;
      acc *= a;
      ctot *= a;
      M = Mn;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float c = (mv[u] > -INFINITY) ? fast_exp2((mv[u] - M) * kLog2e) * ev[u] : 0.f;
        acc += c * v[u];
        ctot += c;
      }
    }
  }
  // Merge the triples of one slice position: lanes f4, f4 + F4, ... of a wave
  // by xor-shuffles, then the waves through LDS.
#pragma unroll
  for (int o = F4; o < 64; o <<= 1) {
    f32x4 ao;
#pragma unroll
    for (int i = 0; i < 4; ++i) ao[i] = __shfl_xor(acc[i], o);
    merge_triple(M, ctot, acc, __shfl_xor(M, o), __shfl_xor(ctot, o), ao);
  }
  if (lane < F4) {
    sm_m[wv][lane] = M;
    sm_c[wv][lane] = ctot;
    sm_a[wv][lane] = acc;
  }
  __syncthreads();
  if (t < F4) {
    M = sm_m[0][t];
    ctot = sm_c[0][t];
    acc = sm_a[0][t];
#pragma unroll
    for (int w = 1; w < NWV; ++w) merge_triple(M, ctot, acc, sm_m[w][t], sm_c[w][t], sm_a[w][t]);
    const float inv = (ctot > 0.f) ? 1.f / ctot : 0.f;
    T* row = reinterpret_cast<T*>(R.out) + (int64_t)sh * R.D + dc * CW;
    store4<T>(row, 4 * t, acc * inv);
  }
}


// ---------------------------------------------------------------- host side
constexpr int kNW = 4;  // waves per f32 partition workgroup
constexpr int kMaxNW = 8;

int partition_size(const pa_shape* sh) { return sh->partition_size ? sh->partition_size : kPart; }

int64_t max_partitions(const pa_shape* sh) {
  const int64_t ps = partition_size(sh);
  return ((int64_t)sh->max_blocks_per_seq * kBS + ps - 1) / ps;
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
  if (wgs * kMaxNW * 64 >= (int64_t)1 << 31) return PA_EUNSUPPORTED;
  if ((int64_t)sh->num_seqs * sh->num_heads * (sh->head_dim / kReduceChunk) * kReduceThreads >= (int64_t)1 << 31)
    return PA_EUNSUPPORTED;
  return PA_OK;
}

// Dynamic LDS: [per-wave max | exp-sum][merge rows [wave][head][D + 4]
// floats], followed (16-bit caches) by the per-wave K tiles.
size_t merge_bytes(int nw, int D, int G) {
  return ((size_t)2 * nw * 16 + (size_t)nw * G * (D + 4)) * sizeof(float);
}


// One launch shape of the 16-bit partition kernel: NW waves per workgroup,
// TB blocks per tile, NBUF tiles in flight per wave, CT tiles per unrolled
// chunk, WPE waves per SIMD.
template <int NW_, int TB_, int NBUF_, int CT_, int WPE_>
struct Shape16 {
  static constexpr int NW = NW_, TB = TB_, NBUF = NBUF_, CT = CT_, WPE = WPE_;
};

template <typename T, int D, typename S>
hipError_t launch_h16(const Params& P, bool trace, dim3 grid, const Launch& L) {
  const size_t ktiles = (size_t)S::NW * S::TB * 16 * D * sizeof(T);
  const size_t smem = merge_bytes(S::NW, D, P.G) + ktiles;
  const size_t max_smem = merge_bytes(S::NW, D, 16) + ktiles;
  if (trace)
    return launch_lds<pa_partition_h16<T, D, S::NW, S::TB, S::NBUF, S::CT, S::WPE, true>>(max_smem, grid, dim3(S::NW * 64),
                                                                                    smem, L, P);
  return launch_lds<pa_partition_h16<T, D, S::NW, S::TB, S::NBUF, S::CT, S::WPE, false>>(max_smem, grid, dim3(S::NW * 64),
                                                                                   smem, L, P);
}

template <int D>
hipError_t launch_f32(const Params& P, bool trace, dim3 grid, const Launch& L) {
  const size_t smem = merge_bytes(kNW, D, P.G);
  const size_t max_smem = merge_bytes(kNW, D, 16);
  if (trace) return launch_lds<pa_partition_f32<D, kNW, true>>(max_smem, grid, dim3(kNW * 64), smem, L, P);
  return launch_lds<pa_partition_f32<D, kNW, false>>(max_smem, grid, dim3(kNW * 64), smem, L, P);
}

// Launch shapes of the 16-bit kernel, chosen from sizes alone (no device
// data is read on the host).
//   head_dim 128:
//     single-pass only (mode V1, or a table no wider than the V1 threshold):
//       few long workgroups -> 8 waves, two-block tiles;
//     at most one workgroup per CU: every workgroup streams on a CU of its
//       own, bound by the CU's load rate, so each wave keeps two one-block
//       tiles in flight (2 waves per SIMD is all such a grid occupies);
//     up to kSmallGrid workgroups: one-block tiles, one in flight (with a
//       deeper ring the first workgroup on a CU takes the CU's load queue
//       and the second one starts late: 100K tokens, 392 workgroups, 20.9
//       against 21.8-22.2 us);
//     otherwise (batches) one-block tiles, two in flight, 3 waves per SIMD:
//       on 64 mixed sequences the long single-pass items stream faster with
//       two tiles in flight (partition kernel 180 against 197 us with
//       two-block tiles and one in flight).
//   head_dim 256: single-pass only -> 4 waves; otherwise 2 waves (more
//     independent workgroups per CU; on 256 sequences of 1K-32K tokens 2.8%
//     faster than 4 waves, which stream one long context faster).
using ShapeV1D128 = Shape16<8, 2, 1, 8, 3>;
using ShapeRingD128 = Shape16<4, 1, 2, 8, 2>;
using ShapeSmallD128 = Shape16<4, 1, 1, 8, 3>;
using ShapeD128 = Shape16<4, 1, 2, 8, 3>;
using ShapeV1D256 = Shape16<4, 1, 1, 8, 2>;
using ShapeD256 = Shape16<2, 1, 1, 16, 2>;
constexpr int64_t kSmallGrid = 1024;

// Compute units of the current device (queried once per device).
int64_t device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool single_pass_grid(const Params& P) {
  return P.mode == PA_MODE_V1 || (P.mode == PA_MODE_AUTO && (int64_t)P.MB * kBS <= kThresh);
}

template <typename T>
hipError_t launch_h16_d128(const Params& P, bool trace, dim3 grid, const Launch& L) {
  if (single_pass_grid(P)) return launch_h16<T, 128, ShapeV1D128>(P, trace, grid, L);
  if ((int64_t)grid.x <= device_cus()) return launch_h16<T, 128, ShapeRingD128>(P, trace, grid, L);
  if ((int64_t)grid.x <= kSmallGrid) return launch_h16<T, 128, ShapeSmallD128>(P, trace, grid, L);
  return launch_h16<T, 128, ShapeD128>(P, trace, grid, L);
}

template <typename T>
hipError_t launch_h16_d256(const Params& P, bool trace, dim3 grid, const Launch& L) {
  if (single_pass_grid(P)) return launch_h16<T, 256, ShapeV1D256>(P, trace, grid, L);
  return launch_h16<T, 256, ShapeD256>(P, trace, grid, L);
}

hipError_t launch_partitions(const Params& P, int D, int dtype, bool trace, const Launch& stream) {
  const int64_t pgrid = (P.mode == PA_MODE_V1) ? 1 : P.Pmax;
  const dim3 grid((unsigned)((int64_t)P.S * P.Hkv * pgrid));
  if (grid.x == 0) return nothing_launched(stream);
  if (dtype == PA_BF16) {
    if (D == 128) return launch_h16_d128<__bf16>(P, trace, grid, stream);
    return launch_h16_d256<__bf16>(P, trace, grid, stream);
  }
  if (dtype == PA_F16) {
    if (D == 128) return launch_h16_d128<_Float16>(P, trace, grid, stream);
    return launch_h16_d256<_Float16>(P, trace, grid, stream);
  }
  if (D == 128) return launch_f32<128>(P, trace, grid, stream);
  return launch_f32<256>(P, trace, grid, stream);
}

// Slice width of the reduce: the widest (fewest workgroups) that still gives
// at least kReduceMinWGs workgroups, 32 floats at the narrowest.
constexpr int64_t kReduceMinWGs = 2048;

// Partial sets up to this size (tmp_out bytes) are reduced with speculative
// first loads: the kernel is then latency-bound and the loads it may waste
// (partitions past a short sequence's end) are few.
constexpr int64_t kReduceSpecBytes = 8 << 20;

template <typename T, int CW>
hipError_t launch_reduce_cw(bool spec, dim3 grid, dim3 block, const Launch& L, const ReduceParams& R) {
  if (spec) return launch(pa_lse_reduce_kernel<T, CW, true>, grid, block, 0, L, R);
  return launch(pa_lse_reduce_kernel<T, CW, false>, grid, block, 0, L, R);
}

template <typename T>
hipError_t launch_reduce_t(const ReduceParams& R, const Launch& L) {
  const int64_t rows = (int64_t)R.S * R.H;
  int cw = 32;
  for (int c : {256, 128, 64}) {
    if (c <= R.D && rows * (R.D / c) >= kReduceMinWGs) {
      cw = c;
      break;
    }
  }
  const dim3 grid((unsigned)(rows * (R.D / cw)));
  if (grid.x == 0) return nothing_launched(L);
  const dim3 block(kReduceThreads);
  const bool spec = rows * R.Pmax * R.D * (int64_t)sizeof(float) <= kReduceSpecBytes;
  switch (cw) {
    case 256: return launch_reduce_cw<T, 256>(spec, grid, block, L, R);
    case 128: return launch_reduce_cw<T, 128>(spec, grid, block, L, R);
    case 64: return launch_reduce_cw<T, 64>(spec, grid, block, L, R);
    default: return launch_reduce_cw<T, 32>(spec, grid, block, L, R);
  }
}

hipError_t launch_reduce(const ReduceParams& R, int dtype, const Launch& L) {
  if (dtype == PA_BF16) return launch_reduce_t<__bf16>(R, L);
  if (dtype == PA_F16) return launch_reduce_t<_Float16>(R, L);
  return launch_reduce_t<float>(R, L);
}

// No sequence can take the partitioned path: V1 forced, or AUTO with a table
// too narrow for any context to pass the threshold (lengths are clamped to
// the table's width).
bool single_pass_only(const pa_shape* sh, int mode) {
  return mode == PA_MODE_V1 || (mode == PA_MODE_AUTO && (int64_t)sh->max_blocks_per_seq * kBS <= kThresh);
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
  P.Pmax = (int)max_partitions(sh); P.mode = mode; P.PS = partition_size(sh);
  // One sequence, or single-pass only: the direct (partition, sequence, KV
  // head) order is already compact. Very large batches keep it too: every
  // workgroup of a compact grid scans all sequence lengths.
  P.compact = !single_pass_only(sh, mode) && P.S > 1 && P.S <= kCompactMaxSeqs && P.Pmax > 1;
  P.scale2 = scale * kLog2e;
  return P;
}

ReduceParams make_reduce_params(void* out, const float* es, const float* ml, const float* to,
                                const int32_t* sl, const pa_shape* sh, int mode) {
  ReduceParams R;
  R.out = out; R.exp_sums = es; R.max_logits = ml; R.tmp_out = to; R.sl = sl;
  R.S = sh->num_seqs; R.H = sh->num_heads; R.MB = sh->max_blocks_per_seq;
  R.Pmax = (int)max_partitions(sh); R.mode = mode; R.D = sh->head_dim; R.PS = partition_size(sh);
  return R;
}


int run_partitions(void* out, const void* q, const void* k, const void* v, const int32_t* bt,
                   const int32_t* sl, const pa_shape* sh, float scale, float* es, float* ml,
                   float* to, int mode, int32_t* trace, int32_t* err, const Launch& L) {
  const int st = check_all(out, q, k, v, bt, sl, sh, es, ml, to, mode, mode != PA_MODE_V1, true);
  if (st != PA_OK) return st;
  (void)hipGetLastError();
  const Params P = make_params(out, q, k, v, bt, sl, sh, scale, es, ml, to, mode, trace, err);
  if (launch_partitions(P, sh->head_dim, sh->dtype, trace != nullptr || err != nullptr, L) != hipSuccess)
    return PA_EHIP;
  return PA_OK;
}

int run_reduce(void* out, const float* es, const float* ml, const float* to, const int32_t* sl,
               const pa_shape* sh, int mode, const Launch& L) {
  const int st = check_all(out, nullptr, nullptr, nullptr, nullptr, sl, sh, es, ml, to, mode, true, false);
  if (st != PA_OK) return st;
  (void)hipGetLastError();
  if (single_pass_only(sh, mode))  // nothing is partitioned
    return nothing_launched(L) == hipSuccess ? PA_OK : PA_EHIP;
  const ReduceParams R = make_reduce_params(out, es, ml, to, sl, sh, mode);
  if (launch_reduce(R, sh->dtype, L) != hipSuccess) return PA_EHIP;
  return PA_OK;
}

int run_full(void* out, const void* q, const void* k, const void* v, const int32_t* bt,
             const int32_t* sl, const pa_shape* sh, float scale, float* es, float* ml, float* to,
             int mode, void* stream) {
  const int st = check_all(out, q, k, v, bt, sl, sh, es, ml, to, mode, mode != PA_MODE_V1, true);
  if (st != PA_OK) return st;
  int rc = run_partitions(out, q, k, v, bt, sl, sh, scale, es, ml, to, mode, nullptr, nullptr, on(stream));
  if (rc != PA_OK || single_pass_only(sh, mode)) return rc;
  return run_reduce(out, es, ml, to, sl, sh, mode, on(stream));
}

}  // namespace

// Partials of pa_decode_noalloc: one array per GPU, owned by the library for
// the life of the process. Host code never names it directly (in host code
// the name is a stand-in, not a device address): scratch_base() returns its
// address on the current device.
static __device__ __align__(256) float scratch[PA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept; nullptr if
// the lookup fails.
float* scratch_base() {
  static std::mutex mu;
  static float* base[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!base[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    base[dev] = static_cast<float*>(p);
  }
  return base[dev];
}

// Offsets (floats) of exp_sums, max_logits and tmp_out in the scratch array
// for a shape, each 256-byte aligned; false when they do not fit.
bool scratch_layout(const pa_shape* sh, int64_t& off_ml, int64_t& off_to) {
  const int64_t n = (int64_t)sh->num_seqs * sh->num_heads * max_partitions(sh);
  const int64_t a = (n + 63) / 64 * 64;
  off_ml = a;
  off_to = 2 * a;
  return off_to + n * sh->head_dim <= (int64_t)(PA_NOALLOC_SCRATCH_BYTES / sizeof(float));
}

}  // namespace

extern "C" {

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* seq_lens, const pa_shape* shape,
                      float scale, void* stream) {
  // validate as pa_decode does, except for the partials (the library's own,
  // aligned), then check that they fit
  const int st = check_all(out, q, k_cache, v_cache, block_tables, seq_lens, shape, nullptr, nullptr, nullptr,
                           PA_MODE_AUTO, false, true);
  if (st != PA_OK) return st;
  if (shape->num_seqs == 0) return PA_OK;
  int64_t off_ml = 0, off_to = 0;
  if (!single_pass_only(shape, PA_MODE_AUTO) && !scratch_layout(shape, off_ml, off_to)) return PA_ESCRATCH;
  float* base = scratch_base();
  if (!base) return PA_EHIP;
  return run_full(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, base, base + off_ml,
                  base + off_to, PA_MODE_AUTO, stream);
}

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
                        max_logits, tmp_out, mode, nullptr, nullptr, on(stream));
}

int pa_lse_reduce(void* out, const float* exp_sums, const float* max_logits, const float* tmp_out,
                  const int32_t* seq_lens, const pa_shape* shape, int mode, void* stream) {
  return run_reduce(out, exp_sums, max_logits, tmp_out, seq_lens, shape, mode, on(stream));
}

int pa_decode_partitions_timed(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               const pa_shape* shape, float scale, float* exp_sums,
                               float* max_logits, float* tmp_out, int mode, void* start_event,
                               void* stop_event, void* stream) {
  return run_partitions(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, exp_sums,
                        max_logits, tmp_out, mode, nullptr, nullptr,
                        Launch{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event});
}

int pa_lse_reduce_timed(void* out, const float* exp_sums, const float* max_logits, const float* tmp_out,
                        const int32_t* seq_lens, const pa_shape* shape, int mode, void* start_event,
                        void* stop_event, void* stream) {
  return run_reduce(out, exp_sums, max_logits, tmp_out, seq_lens, shape, mode,
                    Launch{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event});
}

int pa_decode_partitions_debug(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               const pa_shape* shape, float scale, float* exp_sums,
                               float* max_logits, float* tmp_out, int mode,
                               int32_t* gather_trace, int32_t* err_flag, void* stream) {
  if (gather_trace && !aligned(gather_trace, 4)) return PA_EALIGN;
  if (err_flag && !aligned(err_flag, 4)) return PA_EALIGN;
  return run_partitions(out, q, k_cache, v_cache, block_tables, seq_lens, shape, scale, exp_sums,
                        max_logits, tmp_out, mode, gather_trace, err_flag, on(stream));
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
    case PA_ESCRATCH: return "partials larger than the library's scratch (pa_decode_noalloc; use pa_decode)";
    default: return "unknown status";
  }
}

int pa_version(void) { return 1; }

}  // extern "C"
