// Prefix / chunked-prefill attention over the paged cache for gfx950 (MI355X):
// the kernel and its C ABI entry point (pa_prefill, declared in pa_decode.h).

#include <algorithm>
#include <cfloat>
#include <type_traits>
#include <utility>

#include "pa_common.h"

namespace {

// ---------------------------------------------------------------- prefix / chunked prefill
// Attention of a chunk of query tokens over the paged cache (project_6 commit
// cd0d9e1a, "paged_attn.py rewrite" item 1 and the Triton prefill note: the
// context's K/V come from the cache, query tiles walk key tiles with the
// online softmax; project_6 blame of optimizations/prefix_prefill_patch.py:
// query tiles against key/value tiles, head_dim 128/256, GQA, fp16/bf16).
// Sequence s keeps L tokens in the cache, the last Q of them the chunk; chunk
// token i sits at position L - Q + i and sees cached tokens 0 .. L - Q + i.
//
// The decode tile layout carries over with query rows on the MFMA N axis: a
// row is one (chunk token, query head of the GQA group), row = token * G +
// head, so one K/V tile serves every head of the group and QT tokens. One
// workgroup takes (sequence, KV head, QT-token query tile). Its NW waves
// form KS key groups of NW / KS row groups; each wave owns NTW N-tiles of
// 16 rows and, of every KS consecutive key tiles, the one of its key group
// (with KS = 2 the two key groups merge their partial results at the end).
// The workgroup loads each K/V tile once, straight from memory into LDS,
// and every wave reads its MFMA operands there (K row-permuted so the
// token-wise operand reads hit distinct banks, V read back transposed). P is
// the QK accumulator rounded to the 16-bit type; its row sums come from one
// more MFMA against a ones operand. Outputs are stored straight from the
// accumulators.
// Max over the four lane groups (lanes l, l^16, l^32, l^48: the same row)
// with the gfx950 lane-swap moves instead of LDS-routed shuffles.
// v_permlane16_swap a, b exchanges rows 1/3 of a with rows 0/2 of b; with b a
// copy of a, lane l then holds v[l] and v[l^16] across a and b, and
// v_permlane32_swap pairs l with l^32 the same way. The max of a and b is
// then the same value in both lanes of a pair. The maxima are taken inside
// the assembly too: the inputs are MFMA results or -inf, never signalling
// NaNs, so they need none of the canonicalizing moves the compiler puts
// around a max of values it cannot see the origin of.
// Written as inline assembly with both registers read-write: the compiler's
// builtin for these swaps returned the first result in place of the second
// when both inputs held the same value. The s_nop pairs cover the VALU ->
// lane-swap -> VALU data hazards.
__device__ __forceinline__ float rows_max(float x) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(x), "=&v"(t));
  return x;
}

// gfx950 LDS transpose read of 16-bit data. Within each group of 16 lanes,
// lane j reads 4 consecutive elements in[j][0..3] at its own address; lane i
// receives out[i][e] = in[4e + i/4][i % 4]. So if lane j points at row
// r0 + j/4, columns c0 + 4(j % 4) .. +3 of a row-major matrix, lane i gets
// column c0 + i of rows r0 .. r0 + 3: the A operand layout of a 16x16 MFMA
// (row = lane % 16, four consecutive k) read straight from row-major data.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(const_cast<void*>(p)));
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1, in order.
template <typename F, int... I>
__device__ __forceinline__ void unrolled_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unrolled(F& f) {
  unrolled_impl(f, std::make_integer_sequence<int, N>{});
}

// Runs one step's loads into LDS (fetch) and its math (math) with the LDS
// slots as restrict pointers: the slot a step loads into is never the slot
// its math reads. Inlined, the restrict parameters tag every LDS access
// with alias scopes, which lets the compiler see that the math's reads do
// not depend on the loads in flight (without them it waits for every
// outstanding load before each LDS read).
template <typename Fetch, typename Math>
__device__ __forceinline__ void with_slots(u32x4* __restrict__ k_next, u32x4* __restrict__ v_next,
                                           const u32x4* __restrict__ k_cur, const u32x4* __restrict__ v_cur,
                                           Fetch& fetch, Math& math) {
  fetch(k_next, v_next);
  math(k_cur, v_cur);
}

// Workgroup barrier for LDS written by loads: waits until at most N loads
// of this wave are outstanding and its LDS accesses are done, then
// s_barrier. (A workgroup fence would wait for every load that writes
// LDS, the ones still prefetching included.) The memory clobber keeps the
// compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void lds_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));  // vmcnt(N) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Most 16-byte loads one lane makes per K (or V) tile in any launch shape.
constexpr int kMaxLoadsPerTile = 4;

// Growth of a row's max (log2 units) below which the online softmax keeps
// its reference max: P stays below 2^8.
constexpr float kLazyRescale = 8.f;

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* bt;
  const int32_t* sl;
  const int32_t* qsl;
  void* out;
  int64_t NB;
  int S, H, Hkv, G, MB, T, QT;
  float scale2;
};

// Reduction over the wave with DPP moves: shifts by 1, 2, 4 and 8 lanes
// within each row of 16 leave the row's result in its lane 15, then the
// row broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3)
// combine the rows in lane 63. Lanes without a source keep `id`.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_reduce(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Work item (sequence s, query tile t) of rank g when the items are ordered
// by decreasing cost, ties by increasing s; s = -1 past the last item. The
// cost of an item is the number of keys its last row sees, L - Q + min((t +
// 1) QT, Q), which grows with t within a sequence. Up to 64 SLOTS
// sequences, sequence s in slot s / 64 of lane s % 64. Keys are shifted by T
// so that none is negative (a chunk longer than its sequence has tiles that
// see no key). F(c), the number of items with key >= c, has a closed form
// per sequence and is summed over the slots and the wave; the rank-g key is
// the largest c with F(c) > g, found by bisection, and each sequence has at
// most one item of that key.
constexpr int kRankedSeqs = 256;  // batches up to this size launch in ranked order (4 sequences per lane)

struct WorkItem {
  int s, t;  // s = -1: no item; s = -2: every sequence has the same prefix (take the round order)
};

// A sequence's extents, clamped so that no data value can send a read out of
// bounds: chunk tokens [qb, qb + Q) of q and out, L keys in its block table.
struct SeqExtent {
  int qb, Q, L;
};

__device__ __forceinline__ SeqExtent load_extent(const PrefillParams& P, int s) {
  const int qb_raw = P.qsl[s], qe_raw = P.qsl[s + 1], L_raw = P.sl[s];
  const int qb = min(max(qb_raw, 0), P.T);
  const int qe = min(max(qe_raw, qb), P.T);
  return {qb, qe - qb, min(max(L_raw, 0), P.MB * kBS)};
}

// The extents of sequence s (wave-uniform) from the lane that holds it.
template <int SLOTS>
__device__ __forceinline__ SeqExtent slot_extent(const SeqExtent (&e)[SLOTS], int s) {
  SeqExtent r{0, 0, 0};
#pragma unroll
  for (int k = 0; k < SLOTS; ++k)
    if (k == (s >> 6))
      r = {__builtin_amdgcn_readlane(e[k].qb, s & 63), __builtin_amdgcn_readlane(e[k].Q, s & 63),
           __builtin_amdgcn_readlane(e[k].L, s & 63)};
  return r;
}

template <int SLOTS>
__device__ WorkItem item_by_cost(const PrefillParams& P, const SeqExtent (&e)[SLOTS], int g, int nq, int lane) {
  const int slots = SLOTS == 1 ? 1 : (P.S + 63) / 64;  // 1 .. SLOTS, wave-uniform
  const uint32_t QT = (uint32_t)P.QT;
  uint32_t base[SLOTS], Q[SLOTS], last[SLOTS];
  int n[SLOTS];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    base[k] = Q[k] = 0u;
    n[k] = 0;
    if (k < slots && 64 * k + lane < P.S) {
      base[k] = (uint32_t)e[k].L + ((uint32_t)P.T - (uint32_t)e[k].Q);  // key of the chunk's position 0, shifted by T
      Q[k] = min((uint32_t)e[k].Q, (uint32_t)nq * QT);                  // tiles past the grid's nq are not computed
      n[k] = (int)((Q[k] + QT - 1) / QT);
    }
    last[k] = base[k] + Q[k];  // the key of the sequence's last tile
  }
  auto count_one = [&](int k, uint32_t c) -> uint32_t {  // items of slot k's sequence with key >= c
    if (n[k] == 0 || c > last[k]) return 0u;
    const uint32_t m = ((c > base[k] ? c - base[k] : 0u) + QT - 1) / QT;  // first tile t + 1 whose key is >= c
    return (uint32_t)n[k] + 1u - max(m, 1u);
  };
  auto count = [&](uint32_t c) -> uint32_t {  // this lane's items with key >= c
    uint32_t f = 0;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k)
      if (k < slots) f += count_one(k, c);
    return f;
  };
  // Every sequence alike (a batch of equal prompts): rank g is tile n - 1 -
  // g / S of sequence g % S, with no search. Above 64 sequences, every
  // sequence with the same prefix but chunks of different lengths (fresh
  // prompts): an item's cost is then its tile's end, so the order by
  // query-tile rounds is this order already and spares the search (which
  // up to 64 sequences costs about what the round order would lose).
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(base[0]), q0 = __builtin_amdgcn_readfirstlane(Q[0]);
  bool base_differs = false, q_differs = false;
#pragma unroll
  for (int k = 0; k < SLOTS; ++k)
    if (k < slots && 64 * k + lane < P.S) {
      base_differs |= base[k] != b0;
      q_differs |= Q[k] != q0;
    }
  if (__ballot(base_differs) == 0) {
    const bool chunks_differ = __ballot(q_differs) != 0;
    if (SLOTS > 1 && chunks_differ) return {-2, 0};
    if (!chunks_differ) {
      const int n0 = __builtin_amdgcn_readfirstlane(n[0]);
      if (g >= n0 * P.S) return {-1, 0};
      return {g % P.S, n0 - 1 - g / P.S};
    }
  }
  uint32_t nsum = 0, lo_l = ~0u, hi_l = 0u;
#pragma unroll
  for (int k = 0; k < SLOTS; ++k)
    if (k < slots && n[k]) {
      nsum += (uint32_t)n[k];
      lo_l = min(lo_l, base[k] + min(QT, Q[k]));
      hi_l = max(hi_l, last[k]);
    }
  const uint32_t total = wave_sum(nsum);
  if ((uint32_t)g >= total) return {-1, 0};
  // Bounds: F(lo) = total > g and F(hi) = 0 <= g.
  uint32_t lo = wave_reduce(lo_l, ~0u, [](uint32_t a, uint32_t b) { return min(a, b); });
  uint32_t hi = wave_reduce(hi_l, 0u, [](uint32_t a, uint32_t b) { return max(a, b); }) + 1u;
  uint32_t f_hi = 0;
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const uint32_t f = wave_sum(count(mid));
    if (f > (uint32_t)g) {
      lo = mid;
    } else {
      hi = mid;
      f_hi = f;
    }
  }
  // The item is the (g - F(lo + 1))-th, in sequence order (slot by slot,
  // lane by lane), of those with key lo.
  uint32_t j = (uint32_t)g - f_hi;
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    if (k >= slots) break;
    const bool has = count_one(k, lo) != count_one(k, lo + 1u);
    const uint64_t hm = __ballot(has);
    const uint32_t cnt = (uint32_t)__builtin_popcountll(hm);
    if (j < cnt) {
      const uint32_t below = (uint32_t)__builtin_popcountll(hm & ((1ull << lane) - 1ull));
      const int sel = __builtin_ctzll(__ballot(has && below == j));
      const uint32_t sb = __builtin_amdgcn_readlane(base[k], sel), sl = __builtin_amdgcn_readlane(last[k], sel);
      const int sn = __builtin_amdgcn_readlane(n[k], sel);
      return {64 * k + sel, lo == sl ? sn - 1 : (int)((lo - sb) / QT) - 1};
    }
    j -= cnt;
  }
  return {-1, 0};  // unreachable: F counts exactly the items above
}

// Workgroup blockIdx.x's item: sequence, KV head, query tile and the
// sequence's extents (s = -1: none).
struct Item {
  int s, kvh, qt;
  SeqExtent e;
};

// Round r = b / pairs takes query tile nq - 1 - r of every (sequence, KV
// head) pair, the pairs rotated by r.
__device__ __forceinline__ Item round_order_item(const PrefillParams& P, int nq) {
  const int pairs = P.S * P.Hkv;
  const int r = (int)(blockIdx.x / pairs);
  const int pair = ((int)(blockIdx.x % pairs) + r) % pairs;
  return {pair / P.Hkv, pair % P.Hkv, nq - 1 - r, {0, 0, 0}};
}

// The ranked item (or the round order where item_by_cost defers to it), with
// the extents read from the lanes that loaded them for the search: no
// second round trip to memory.
template <int SLOTS>
__device__ __forceinline__ Item find_item(const PrefillParams& P, int nq, int lane) {
  // Every slot loads (sequence index clamped into the batch, S >= 1) and the
  // lanes past the batch drop theirs afterwards: the loads of all slots go
  // out together, where a load under a per-slot branch would wait for its
  // own round trip.
  SeqExtent e[SLOTS];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) e[k] = load_extent(P, min(64 * k + lane, P.S - 1));
#pragma unroll
  for (int k = 0; k < SLOTS; ++k)
    if (64 * k + lane >= P.S) e[k] = {0, 0, 0};
  const WorkItem w = item_by_cost<SLOTS>(P, e, (int)(blockIdx.x / P.Hkv), nq, lane);
  if (w.s == -1) return {-1, 0, 0, {0, 0, 0}};
  Item it = w.s >= 0 ? Item{w.s, (int)(blockIdx.x % P.Hkv), w.t, {0, 0, 0}} : round_order_item(P, nq);
  it.e = slot_extent(e, it.s);
  return it;
}

template <typename T, int D, int NW, int NTW, int TB, int SHD, int KS>
__global__ __launch_bounds__(NW * 64, 2) void pa_prefill_h16(PrefillParams P) {
  typedef typename H16<T>::x8 tx8;
  extern __shared__ float smem[];
  constexpr int KK = D / 32;    // QK MFMAs per block and N-tile
  constexpr int NACC = D / 16;  // output tiles (16 head dims each) per N-tile
  constexpr int KCH = D / 8;    // 16-byte chunks per head_dim row
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15, grp = lane >> 4;
  // Key split: the waves form KS groups of NW / KS; wave w takes row group
  // w % (NW / KS) and, of every KS consecutive key tiles, tile w / (NW / KS).
  static_assert(NW % KS == 0, "key groups of equal size");
  // Loads per lane into LDS: K and V tiles of TB blocks of 16 rows of D / 8
  // 16-byte chunks, spread over the NW x 64 lanes (NLD per tile each), KS
  // tiles per step.
  constexpr int NLD = TB * 16 * (D / 8) / (NW * 64);
  static_assert(NLD >= 1 && NLD <= kMaxLoadsPerTile && NLD * NW * 64 == TB * 16 * (D / 8), "whole loads per tile");
  constexpr int kLoadsPerStep = 2 * KS * NLD;
  constexpr int NWR = NW / KS;  // waves per key group (row groups)
  const int rg = w % NWR, kg = w / NWR;

  // Launch order. The CUs take workgroups in launch order as they free up, so
  // the order is the schedule: the items that see the most keys go first and
  // the short ones fill the tail. With up to kRankedSeqs sequences (above 64,
  // only when their prefix lengths differ), workgroup b takes KV head b % Hkv
  // of the item of rank b / Hkv by cost (item_by_cost: exact, whatever the
  // prefix and chunk lengths). Otherwise round r = b / pairs takes query tile
  // nq - 1 - r of every (sequence, KV head) pair (the later tiles of a chunk
  // see the most keys; with equal prefixes that is the order by cost), the
  // pairs rotated by r: workgroups go to the XCDs round-robin, and without the
  // rotation each XCD would take the same few pairs in every round.
  const int nq = (int)(gridDim.x / (P.S * P.Hkv));
  const Item it = P.S <= 64 ? find_item<1>(P, nq, lane) : P.S <= kRankedSeqs ? find_item<4>(P, nq, lane) : [&] {
    Item r = round_order_item(P, nq);
    r.e = load_extent(P, r.s);
    return r;
  }();
  if (it.s < 0) return;
  const int s = it.s, kvh = it.kvh, qt = it.qt;
  const int qb = it.e.qb, Q = it.e.Q, L = it.e.L;
  const int i0 = qt * P.QT;
  if (i0 >= Q) return;
  const int i1 = min(i0 + P.QT, Q);
  const int base = L - Q;                   // position of chunk token 0 (negative: no keys)
  const int kmax = min(L, base + i1);       // the tile's rows see keys [0, kmax)

  // This lane's row in each of the wave's N-tiles.
  int tokr[NTW], posc[NTW];
  bool valid[NTW], live[NTW];
#pragma unroll
  for (int jj = 0; jj < NTW; ++jj) {
    const int row = (rg * NTW + jj) * 16 + g;
    const int tok = i0 + row / P.G;
    valid[jj] = row < P.QT * P.G && tok < i1;
    tokr[jj] = tok;
    const int pos = base + tok;
    live[jj] = valid[jj] && pos >= 0;
    posc[jj] = live[jj] ? pos : kmax - 1;   // rows without keys compute a harmless stand-in
  }
  // Smallest position among the wave's rows: key tiles that end at or below
  // it need no causal mask (every row sees every key of the tile).
  int min_pos = posc[0];
#pragma unroll
  for (int jj = 1; jj < NTW; ++jj) min_pos = min(min_pos, posc[jj]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) min_pos = min(min_pos, __shfl_xor(min_pos, o));
  const int wave_min_pos = __builtin_amdgcn_readfirstlane(min_pos);
  auto out_row = [&](int jj) -> T* {
    const int row = (rg * NTW + jj) * 16 + g;
    return reinterpret_cast<T*>(P.out) + ((int64_t)(qb + tokr[jj]) * P.H + kvh * P.G + row % P.G) * D;
  };

  if (kmax <= 0) {  // no row of the tile sees a key
#pragma unroll
    for (int jj = 0; jj < NTW; ++jj)
      if (valid[jj] && grp == 0)
        for (int d = 0; d < D; d += 4) store4<T>(out_row(jj), d, (f32x4){0.f, 0.f, 0.f, 0.f});
    return;
  }

  // B operands of the QK MFMA: lane holds q[row][kk*32 + 8*grp .. +8].
  // A negative scale is folded into q (an exact sign flip), so that the
  // softmax below scales by |scale| and takes its running max on the raw
  // scores (the max commutes with a non-negative scale). A zero scale is
  // folded in as q = 0 with scale 1: every score is then exactly 0, and
  // every visible key weighs exactly 1, as with the zero scale itself; the
  // softmax thus always scales by a positive number, which sends masked
  // scores (-inf) to exactly 0.
  const bool neg_scale = P.scale2 < 0.f, zero_scale = P.scale2 == 0.f;
  const float s2 = zero_scale ? 1.f : fabsf(P.scale2);
  tx8 qv[NTW][KK];
#pragma unroll
  for (int jj = 0; jj < NTW; ++jj) {
    const int row = (rg * NTW + jj) * 16 + g;
    const T* qrow = reinterpret_cast<const T*>(P.q) +
                    ((int64_t)(qb + tokr[jj]) * P.H + kvh * P.G + row % P.G) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid[jj]) x = ld16(qrow + kk * 32 + grp * 8);
      if (neg_scale) x ^= (u32x4){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      if (zero_scale) x = (u32x4){0u, 0u, 0u, 0u};
      qv[jj][kk] = __builtin_bit_cast(tx8, x);
    }
  }

  const int64_t head_elems = (int64_t)kBS * D;
  const int64_t block_elems = head_elems * P.Hkv;
  const T* kbase = reinterpret_cast<const T*>(P.k) + kvh * head_elems;
  const T* vbase = reinterpret_cast<const T*>(P.v) + kvh * head_elems;
  const int32_t* bt_row = P.bt + (int64_t)s * P.MB;
  const int nblk = (kmax + kBS - 1) / kBS;
  const int ntiles = (nblk + TB - 1) / TB;

  // Running max (log2 units of the scaled scores), P.V accumulators, and
  // the row sums of P: one more MFMA per tile multiplies P by a ones
  // operand, so every lane ends with its row's sum of the same rounded P
  // that the P.V products used (and the vector ALU adds nothing up).
  float m[NTW];
  f32x4 acc[NTW][NACC], accl[NTW];
#pragma unroll
  for (int jj = 0; jj < NTW; ++jj) {
    m[jj] = -INFINITY;
    accl[jj] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[jj][a] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  tx8 ones8;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones8[i] = (T)1.0f;

  auto pack_p2 = [&](const T (&p0)[4], const T (&p1)[4]) {  // two blocks of P as one B operand, keys 4grp+i, 16+4grp+i
    tx8 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = p0[i];
      pv[4 + i] = p1[i];
    }
    return pv;
  };

  {
    // The workgroup loads each K/V tile once into LDS and every
    // wave reads its MFMA operands there. The loads go straight from memory
    // into LDS (buffer loads with the LDS flag: a wave's 64 lanes write 1 KB
    // at the wave's LDS address, lane L at +16 L), so no registers stage the
    // tiles and no stores move them. LDS rows are the KCH 16-byte chunks of
    // a head_dim row, permuted by row so that both operand reads are free of
    // bank conflicts: K row r keeps chunk c at position c ^ (r % 16) (the 16
    // rows a K read takes hit 16 distinct positions mod 16); V row r keeps
    // chunk c at c ^ 2 (r % 8) (the transpose read takes chunk pairs 2mt,
    // 2mt+1 from rows 4grp .. 4grp+3, and eight consecutive rows then hit
    // eight distinct 32-byte bank groups). Each lane loads the global chunk
    // that its LDS position holds. A tile is four blocks of 16 keys; the P.V
    // products take them in two pairs (16x16x32 MFMAs).
    static_assert(KCH == 16 || KCH == 32, "head_dim 128 or 256");
    constexpr int TCH = TB * 16 * KCH;               // chunks per K (or V) tile
    constexpr int RPW = 64 / KCH;                    // tile rows one load of a wave covers
    static_assert(TB == 4 && ((D == 128 && NTW == 2) || (D == 256 && NTW == 1)), "the launch shapes' tiles");
    struct PV {                                       // P as the B operands of the P.V products
      tx8 p[2];                                       // block pairs 0 and 1
    };
    // LDS: NSL slots (step % NSL) of KS tiles each, K [NSL][KS][TB*16][KCH]
    // then V [NSL][KS][TB*16][KCH]. A step is KS consecutive key tiles, one
    // per key group. Steps σ + 1 .. σ + SHD load while step σ is computed:
    // SHD + 1 slots, and the loop runs in groups of NSL so that every slot
    // index is a compile-time constant.
    static_assert(SHD >= 1, "a step in flight");
    constexpr int NSL = SHD + 1;
    u32x4* kst = reinterpret_cast<u32x4*>(smem);
    u32x4* vst = kst + NSL * KS * TCH;
    // Loads: load i of wave w takes tile rows (w NLD + i) RPW .. + RPW - 1 of
    // each tile of a step, from K and from V. The wave's block of the tile
    // is one block-table entry, read by a scalar load one step ahead; the
    // buffer resources are zero bytes long for blocks past the end, and a V
    // resource ends at the block's last row below kmax (a lane's 16 bytes
    // lie in one row), so those rows arrive as zeros with no per-lane test.
    // Every wave issues the same 2 KS NLD loads per step; a step's loads are
    // waited for (vmcnt, counted by hand: the compiler does not track writes
    // to LDS that come from loads) at the end of the iteration before its
    // math.
    constexpr uint32_t kRowBytes = (uint32_t)(D * sizeof(T));
    constexpr uint32_t kBlockBytes = kBS * kRowBytes;
    const int lp = lane % KCH;                        // LDS position in the row
    // A wave's NLD loads of a tile take NLD x RPW consecutive rows, which lie
    // in one block of the tile (block bw), so one block id and one pair of
    // buffer resources serve them all.
    static_assert(16 % (NLD * RPW) == 0, "a wave's loads of a tile lie in one block");
    const int bw = w * NLD * RPW / 16;
    int wrow[kMaxLoadsPerTile], lrow[kMaxLoadsPerTile], koff[kMaxLoadsPerTile],
        voff[kMaxLoadsPerTile];                       // per load i < NLD
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      wrow[i] = (w * NLD + i) * RPW;                  // first tile row load i writes
      lrow[i] = (wrow[i] + lane / KCH) % 16;          // this lane's row in the block
      koff[i] = (lrow[i] * D + (lp ^ lrow[i]) * 8) * (int)sizeof(T);
      voff[i] = (lrow[i] * D + (lp ^ (2 * (lrow[i] & 7))) * 8) * (int)sizeof(T);
    }
    // The block table through the constant address space: a uniform load
    // from there is a scalar load, waited for by the barrier's counter
    // rather than behind the vector loads in flight.
    const __attribute__((address_space(4))) int32_t* bt_const =
        (const __attribute__((address_space(4))) int32_t*)(uintptr_t)bt_row;
    auto block_id = [&](int u) {                      // physical block of the wave's block of tile u
      const int blk = __builtin_amdgcn_readfirstlane(min(u * TB + bw, nblk - 1));
      int id = bt_const[blk];
      if ((uint64_t)(int64_t)id >= (uint64_t)P.NB) id = 0;  // out-of-range ids read block 0
      return id;
    };
    int id_next[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) id_next[j] = block_id(j);
    auto fetch = [&](int step, u32x4* k_next, u32x4* v_next) {  // the step's tiles into an LDS slot
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int u = step * KS + j;
        const int id = id_next[j];
        id_next[j] = block_id(u + KS);
        const int blk = u * TB + bw;
        const bool ok = blk < nblk;
        const int64_t off = ok ? (int64_t)id * block_elems : 0;
        const uint32_t n = ok ? kBlockBytes : 0u;
        const uint32_t nv = ok ? (uint32_t)min(max(kmax - blk * kBS, 0), kBS) * kRowBytes : 0u;  // rows below kmax
        const __amdgpu_buffer_rsrc_t kr = block_rsrc(kbase + off, n);
        const __amdgpu_buffer_rsrc_t vr = block_rsrc(vbase + off, nv);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int rows = j * TCH + wrow[i] * KCH;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(k_next + rows),
                                                   16, koff[i], 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(v_next + rows),
                                                   16, voff[i], 0, 0, 0);
        }
      }
    };
    int klo[KK];                                      // lane offsets (chunks) of the K operand reads
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) klo[kk] = g * KCH + ((4 * kk + grp) ^ g);
    int vlo[NACC];                                    // lane offsets (bytes) of the V transpose reads
#pragma unroll
    for (int mt = 0; mt < NACC; ++mt) {
      const int R = 4 * grp + (g >> 2);
      vlo[mt] = (R * KCH + 2 * (mt ^ (R & 7)) + ((g >> 1) & 1)) * 16 + (g & 1) * 8;
    }
    auto qk_tile = [&](const u32x4* kt, f32x4 (&sc)[NTW][TB]) {  // QK scores of the K tile at kt
      // The K operands are read one block ahead (two sets of KK registers in
      // turn), the reads of block b + 1 interleaved with the products of
      // block b (sched_group_barrier: one MFMA per N-tile, one LDS read). At
      // head_dim 256 a whole tile's operands would take 128 registers and the
      // compiler read each just before its product and waited on it; at 128
      // it read them all up front (64 registers) and waited on the first.
      tx8 k0[KK], k1[KK];
      auto read_k = [&](int b, tx8 (&ka)[KK]) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) ka[kk] = __builtin_bit_cast(tx8, kt[klo[kk] + b * 16 * KCH]);
      };
      auto mma_k = [&](int b, const tx8 (&ka)[KK]) __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj) sc[jj][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
          for (int jj = 0; jj < NTW; ++jj) sc[jj][b] = H16<T>::mma32(ka[kk], qv[jj][kk], sc[jj][b]);
      };
      read_k(0, k0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        if (b % 2 == 0) {
          mma_k(b, k0);
          if (b + 1 < TB) read_k(b + 1, k1);
        } else {
          mma_k(b, k1);
          if (b + 1 < TB) read_k(b + 1, k0);
        }
        if (b + 1 < TB) {
#pragma unroll
          for (int i = 0; i < KK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, NTW, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // P.V products (and row sums). V^T operand of M-tile mt (head dims
    // 16mt .. 16mt+15) for block pair pp (blocks 2pp, 2pp + 1 of the V tile at
    // vb): keys 4grp .. 4grp+3 of each, in the order the QK accumulator hands
    // P over.
    auto read_v = [&](const char* vb, int pp, tx8 (&vo)[NACC]) __attribute__((always_inline)) {
#pragma unroll
      for (int mt = 0; mt < NACC; ++mt) {
        const i16x4 lo = lds_read_tr16(vb + vlo[mt] + 2 * pp * 16 * KCH * 16);
        const i16x4 hi = lds_read_tr16(vb + vlo[mt] + (2 * pp + 1) * 16 * KCH * 16);
        vo[mt] = __builtin_bit_cast(tx8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto mma_pv = [&](const tx8 (&vo)[NACC], const PV& pv, int jj, int pp) __attribute__((always_inline)) {
#pragma unroll
      for (int mt = 0; mt < NACC; ++mt) acc[jj][mt] = H16<T>::mma32(vo[mt], pv.p[pp], acc[jj][mt]);
      accl[jj] = H16<T>::mma32(ones8, pv.p[pp], accl[jj]);
    };
    // The math of key tile t: QK scores, online-softmax update (running max,
    // rescale of the accumulators), P rounded to the 16-bit type, P.V. The
    // code runs straight through but for two branches: the causal mask, only
    // on tiles that reach past the wave's smallest position (masked scores
    // become -inf), and the rescale, skipped unless some row's max outgrew
    // its reference (rare once the maxima settle). P and the P.V products of
    // both N-tiles are then one basic block, in which the exponentials of one
    // N-tile issue while the matrix cores run the products of the other.
    auto tile_math = [&](const u32x4* kt, const u32x4* vt, int t) __attribute__((always_inline)) {
      f32x4 sc[NTW][TB];
      qk_tile(kt, sc);
      const int tok0 = t * TB * kBS;
      if (tok0 + TB * kBS - 1 > wave_min_pos) {
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj)
#pragma unroll
          for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (tok0 + b * kBS + 4 * grp + i > posc[jj]) sc[jj][b][i] = -INFINITY;
      }
      float mb[NTW], alpha[NTW];
      bool grew = false;
#pragma unroll
      for (int jj = 0; jj < NTW; ++jj) {
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[jj][b][i]);
        mx = rows_max(mx);
        // The reference m (log2 units) moves only when the row's max exceeds
        // it by more than kLazyRescale: P = 2^(score - m) then stays below
        // 2^kLazyRescale, as exact in bf16 and fp16 as below 1, and the
        // rescale of the accumulators is rare after a row's first tiles. A
        // row with no visible key so far keeps m = -inf (with a key split, a
        // key group's first tile can hide every key from a row): alpha is
        // then 1, and P is taken against -FLT_MAX (every score of the row is
        // -inf, so P is still 0).
        const float mt = mx * s2;
        const bool moves = mt > m[jj] + kLazyRescale;
        const float mnew = moves ? mt : m[jj];
        alpha[jj] = moves ? fast_exp2(m[jj] - mnew) : 1.f;
        grew |= moves;
        m[jj] = mnew;
        mb[jj] = fmaxf(mnew, -FLT_MAX);
      }
      if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj) {
#pragma unroll
          for (int a = 0; a < NACC; ++a) acc[jj][a] *= alpha[jj];
          accl[jj] *= alpha[jj];
        }
      }
      PV pv[NTW];
      auto make_p = [&](int jj) __attribute__((always_inline)) {  // P of N-tile jj, as P.V operands
        T pb[TB][4];
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) pb[b][i] = (T)fast_exp2(__builtin_fmaf(sc[jj][b][i], s2, -mb[jj]));
        pv[jj].p[0] = pack_p2(pb[0], pb[1]);
        pv[jj].p[1] = pack_p2(pb[2], pb[3]);
      };
      // Block pairs 0 and 1 in scheduler-fenced phases (sched_barrier), with
      // the issue order inside some set by sched_group_barrier (masks: 0x8
      // MFMA, 0x100 LDS read, 0x402 vector ALU and transcendental): (1) V
      // reads of pair 0 beside P of N-tile 0; with two N-tiles, (2) P.V of
      // N-tile 0, pair 0, one MFMA then five vector instructions of P of
      // N-tile 1 at a time; (3) P.V of the last N-tile, pair 0, one MFMA then
      // two V reads of pair 1 at a time; (4) P.V of pair 1. Left to itself
      // the compiler reads V just before each product and waits on it.
      const char* vb = reinterpret_cast<const char*>(vt);
      tx8 vo0[NACC], vo1[NACC];
      read_v(vb, 0, vo0);
      make_p(0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NTW == 2) {
        mma_pv(vo0, pv[0], 0, 0);
        make_p(1);
#pragma unroll
        for (int i = 0; i < NACC + 1; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mma_pv(vo0, pv[NTW - 1], NTW - 1, 0);
      read_v(vb, 1, vo1);
#pragma unroll
      for (int i = 0; i < NACC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < NTW; ++jj) mma_pv(vo1, pv[jj], jj, 1);
    };
    // Iteration σ (slot σ % NSL) starts the loads of step σ + SHD, runs this
    // wave's tile of the step (QK products, softmax, P.V products), waits
    // for the loads of step σ + 1 and ends with one barrier. The loop runs
    // in whole groups of NSL; iterations past the last step load nothing.
    const int nsteps = (ntiles + KS - 1) / KS;
    {
      auto none = [](const u32x4*, const u32x4*) {};
      auto prologue = [&](auto d_const) {
        constexpr int d = decltype(d_const)::value;
        auto f = [&](u32x4* kn, u32x4* vn) { fetch(d, kn, vn); };
        with_slots(kst + d * KS * TCH, vst + d * KS * TCH, kst + SHD * KS * TCH, vst + SHD * KS * TCH, f, none);
      };
      unrolled<SHD>(prologue);
    }
    lds_barrier<kLoadsPerStep * (SHD - 1)>();  // step 0 is in LDS
    for (int s0 = 0; s0 < nsteps; s0 += NSL) {
      auto iteration = [&](auto d_const) {
        constexpr int d = decltype(d_const)::value;  // == step % NSL
        const int step = s0 + d;
        const int t = step * KS + kg;
        auto load = [&](u32x4* kn, u32x4* vn) { fetch(step + SHD, kn, vn); };
        auto math = [&](const u32x4* kc, const u32x4* vc) {
          if (t < ntiles) tile_math(kc, vc, t);
        };
        constexpr int nx = (d + SHD) % NSL;
        with_slots(kst + nx * KS * TCH, vst + nx * KS * TCH, kst + (d * KS + kg) * TCH, vst + (d * KS + kg) * TCH,
                   load, math);
        lds_barrier<kLoadsPerStep * (SHD - 1)>();  // step σ + 1 is in LDS
      };
      unrolled<NSL>(iteration);
    }
    // Nothing may still land in LDS once it is reused: each wave drains its
    // loads (those past the last step write zeros), then a barrier.
    __builtin_amdgcn_s_waitcnt(0x7 << 4);  // vmcnt(0) lgkmcnt(0)
    if constexpr (KS > 1) __syncthreads();
    if constexpr (KS > 1) {
      // Key groups 1 .. KS-1 hand (max, P.V accumulators, row sums) to key
      // group 0 through LDS (free again after the loop's last barrier), which
      // rescales each to the common max and adds them up. Records are 16
      // bytes per lane, lane-major, so the 16-byte accesses hit distinct banks.
      static_assert(NTW <= 4, "the maxima of a wave's N-tiles share one record");
      constexpr int REC = NTW * (NACC + 1) + 1;      // 16-byte records per lane
      f32x4* mrg = reinterpret_cast<f32x4*>(smem);
      auto at = [&](int k, int e) -> f32x4& { return mrg[(((k - 1) * NWR + rg) * REC + e) * 64 + lane]; };
      if (kg > 0) {
        f32x4 mm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj) {
          mm[jj] = m[jj];
#pragma unroll
          for (int a = 0; a < NACC; ++a) at(kg, jj * (NACC + 1) + a) = acc[jj][a];
          at(kg, jj * (NACC + 1) + NACC) = accl[jj];
        }
        at(kg, NTW * (NACC + 1)) = mm;
      }
      __syncthreads();
      if (kg > 0) return;
#pragma unroll
      for (int k = 1; k < KS; ++k) {
        const f32x4 mm = at(k, NTW * (NACC + 1));
#pragma unroll
        for (int jj = 0; jj < NTW; ++jj) {
          // key group 0 saw key 0, so m[jj] is finite; a group without a
          // visible key has mm = -inf and weighs nothing
          const float mx = fmaxf(m[jj], mm[jj]);
          const float f0 = fast_exp2(m[jj] - mx), f1 = fast_exp2(mm[jj] - mx);
          m[jj] = mx;
#pragma unroll
          for (int a = 0; a < NACC; ++a) acc[jj][a] = acc[jj][a] * f0 + at(k, jj * (NACC + 1) + a) * f1;
          accl[jj] = accl[jj] * f0 + at(k, jj * (NACC + 1) + NACC) * f1;
        }
      }
    }
  }

  // acc[jj][mt][i] holds dim 16mt + 4grp + i of the lane's row; every lane
  // of a row holds its sum.
#pragma unroll
  for (int jj = 0; jj < NTW; ++jj) {
    if (!valid[jj]) continue;
    const float inv = live[jj] ? 1.f / accl[jj][0] : 0.f;
    T* orow = out_row(jj);
#pragma unroll
    for (int mt = 0; mt < NACC; ++mt) store4<T>(orow, 16 * mt + 4 * grp, acc[jj][mt] * inv);
  }
}

// Prefill launch shapes: 8 waves, four-block key tiles (64 keys per step and
// barrier), one step of K/V tiles in flight where the LDS holds only two
// slots of them (measured on the four prefill workloads against other wave,
// N-tile, tile, key-split and prefetch choices; 64-key steps with one step
// in flight beat 32-key steps with two in every shape, 1.07-1.12x):
//   D = 128, at most kPrefillSmallGrid workgroups of 128 rows (long contexts,
//     few query tiles): 4 row groups x 2 N-tiles x 2 key groups, so that 256
//     workgroups still fill the chip with 32-row waves;
//   D = 128, larger grids: 256 rows per workgroup, 8 waves x 2 N-tiles, no
//     key split, two steps in flight (96 KB; 1.02x one step);
//   D = 128, larger grids over tables of at most kPrefillShortTable tokens:
//     128 rows, 4 waves x 2 N-tiles, 64 KB, two workgroups per CU, so that
//     one workgroup's prologue and output stores overlap the other's steps
//     (1.04-1.14x on prompts of up to 1024 tokens, 1.06-1.12x on 128 short
//     chunks behind prefixes of up to 6K tokens, 0.98-1.03x on long chunks
//     in such tables; on longer contexts the 8-wave form, which shares each
//     K/V tile among twice the rows, was 1.03-1.06x faster);
//   D = 256: 128 rows per workgroup, 8 waves x 1 N-tile (the register budget
//     of the wider rows), no key split.
// The P.V products take a tile's four blocks as two pairs, as 16x16x32
// MFMAs (one-block tiles would make them 16x16x16 ones, which do half the
// work in the same issue time).
constexpr int kPrefillRows = 64;       // rows per workgroup: a lower bound over the launch shapes
constexpr int kPrefillMaxNW = 8;       // waves per workgroup, largest launch shape
constexpr int64_t kPrefillSmallGrid = 512;
constexpr int64_t kPrefillShortTable = 8192;

// A launch shape: D, NW waves, NTW N-tiles per wave, TB-block key tiles,
// SHD steps in flight, KS key groups.
template <int D_, int NW_, int NTW_, int TB_, int SHD_, int KS_>
struct PShape {
  static constexpr int D = D_, NW = NW_, NTW = NTW_, TB = TB_, SHD = SHD_, KS = KS_;
};

// Launches shape S: (NW / KS) x NTW x 16 query rows per workgroup, QT = rows
// / G tokens (the last rows % G rows idle when G does not divide them). LDS:
// SHD + 1 slots of KS K and V tiles, or the key groups' merge records (NW /
// KS waves x (NTW (NACC + 1) + 1) x 64 lanes x 16 bytes), whichever is
// larger.
template <typename T, typename S>
hipError_t launch_shape(PrefillParams P, int maxq, const Launch& L) {
  constexpr int rows = S::NW / S::KS * S::NTW * 16;
  static_assert(rows >= kPrefillRows && S::NW <= kPrefillMaxNW, "the grid bound check_prefill applies");
  constexpr size_t tile = (size_t)S::TB * kBS * S::D * sizeof(T);  // one K or V tile
  constexpr size_t slots = (size_t)(S::SHD + 1) * S::KS * 2 * tile;
  constexpr size_t merge =
      S::KS > 1 ? (size_t)(S::KS - 1) * (S::NW / S::KS) * (S::NTW * (S::D / 16 + 1) + 1) * 64 * 16 : 0;
  constexpr size_t smem = slots > merge ? slots : merge;
  static_assert(smem <= 160 * 1024, "LDS of one CU");
  P.QT = rows / P.G;
  const int64_t grid = (int64_t)P.S * P.Hkv * ((maxq + P.QT - 1) / P.QT);
  return launch_lds<pa_prefill_h16<T, S::D, S::NW, S::NTW, S::TB, S::SHD, S::KS>>(
      smem, dim3((unsigned)grid), dim3(S::NW * 64), smem, L, P);
}

template <typename T>
hipError_t launch_prefill_t(PrefillParams P, int D, int maxq, const Launch& L) {
  if (D == 128) {
    const int qt = 128 / P.G;
    if ((int64_t)P.S * P.Hkv * ((maxq + qt - 1) / qt) <= kPrefillSmallGrid)
      return launch_shape<T, PShape<128, 8, 2, 4, 1, 2>>(P, maxq, L);
    if ((int64_t)P.MB * kBS <= kPrefillShortTable) return launch_shape<T, PShape<128, 4, 2, 4, 1, 1>>(P, maxq, L);
    return launch_shape<T, PShape<128, 8, 2, 4, 2, 1>>(P, maxq, L);
  }
  return launch_shape<T, PShape<256, 8, 1, 4, 1, 1>>(P, maxq, L);
}

int check_prefill(const void* out, const void* q, const void* k, const void* v, const int32_t* bt,
                  const int32_t* sl, const int32_t* qsl, const pa_shape* sh, int32_t T, int32_t maxq) {
  const int st = check_shape(sh);
  if (st != PA_OK) return st;
  if (sh->dtype != PA_BF16 && sh->dtype != PA_F16) return PA_EUNSUPPORTED;
  if (T < 0 || maxq < 0) return PA_EINVAL;
  if (sh->num_seqs == 0 || T == 0 || maxq == 0) return PA_OK;  // nothing is read or written
  if (!out || !q || !k || !v || !bt || !sl || !qsl) return PA_EINVAL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(bt, 4) ||
      !aligned(sl, 4) || !aligned(qsl, 4))
    return PA_EALIGN;
  const int G = sh->num_heads / sh->num_kv_heads;
  const int64_t qt = kPrefillRows / G;
  const int64_t wgs = (int64_t)sh->num_seqs * sh->num_kv_heads * ((maxq + qt - 1) / qt);
  if (wgs >= ((int64_t)1 << 31) / (kPrefillMaxNW * 64)) return PA_EUNSUPPORTED;
  if ((int64_t)T * sh->num_heads * sh->head_dim >= ((int64_t)1 << 62)) return PA_EUNSUPPORTED;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
               const int32_t* seq_lens, const int32_t* query_start_loc, const pa_shape* shape,
               int32_t num_query_tokens, int32_t max_query_len, float scale, void* stream) {
  const int st = check_prefill(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, shape,
                               num_query_tokens, max_query_len);
  if (st != PA_OK) return st;
  const Launch L = on(stream);
  if (shape->num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0)
    return nothing_launched(L) == hipSuccess ? PA_OK : PA_EHIP;
  (void)hipGetLastError();
  PrefillParams P;
  P.q = q; P.k = k_cache; P.v = v_cache; P.bt = block_tables; P.sl = seq_lens; P.qsl = query_start_loc;
  P.out = out; P.NB = shape->num_blocks;
  P.S = shape->num_seqs; P.H = shape->num_heads; P.Hkv = shape->num_kv_heads;
  P.G = shape->num_heads / shape->num_kv_heads; P.MB = shape->max_blocks_per_seq;
  P.T = num_query_tokens;
  P.QT = 0;  // set by the launch shape
  P.scale2 = scale * kLog2e;
  const hipError_t e = shape->dtype == PA_BF16 ? launch_prefill_t<__bf16>(P, shape->head_dim, max_query_len, L)
                                               : launch_prefill_t<_Float16>(P, shape->head_dim, max_query_len, L);
  return e == hipSuccess ? PA_OK : PA_EHIP;
}

}  // extern "C"
