// Helpers shared by the attention kernels of this library (decode over the
// paged cache, and prefix/chunked prefill over the same cache): vector types,
// the K/V load forms, the 16-bit MFMA wrappers, the per-wave tile of whole
// 16-token blocks, shape validation and kernel launch with optional events.
// Included by one translation unit each; everything sits in an anonymous
// namespace, so every unit gets its own copy.
#pragma once

#include <atomic>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_decode.h"

namespace {

constexpr int kBS = PA_BLOCK_SIZE;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Loads of the K/V stream (each byte is read once per call) carry the
// non-temporal hint: measured 6-10% faster than plain loads on the largest
// batch (pure reads reach ~6.4 TB/s that way).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
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

// 16-bit element types of the cache: operand vectors and the two MFMA shapes
// the partition kernel uses (16x16x32 for QK and two-block P.V, 16x16x16 for
// one-block P.V). bf16 and fp16 share every lane layout.
template <typename T>
struct H16;
template <>
struct H16<__bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
  static __device__ __forceinline__ f32x4 mma32(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(x4 a, x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b),
                                                      c, 0, 0, 0);
  }
};
template <>
struct H16<_Float16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
  static __device__ __forceinline__ f32x4 mma32(x8 a, x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(x4 a, x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

// Store 4 consecutive head dims starting at dim d of head g.
template <typename T>
__device__ __forceinline__ void store4(T* row, int d, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* row, int d, f32x4 v) {
  *reinterpret_cast<f32x4*>(row + d) = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* row, int d, f32x4 v) {
  bf16x4 b;
  b[0] = (__bf16)v[0];
  b[1] = (__bf16)v[1];
  b[2] = (__bf16)v[2];
  b[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(row + d) = b;
}
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* row, int d, f32x4 v) {
  f16x4 b;
  b[0] = (_Float16)v[0];
  b[1] = (_Float16)v[1];
  b[2] = (_Float16)v[2];
  b[3] = (_Float16)v[3];
  *reinterpret_cast<f16x4*>(row + d) = b;
}

template <int D, int TB>
struct BTile {  // element-type agnostic: raw 16-byte chunks
  static constexpr int NH = D / 128;
  u32x4 k[TB][4][NH];  // K[4*grp + rr][128h + 8g .. +8]
  u32x4 v[TB][4][NH];  // V[4*grp + rr][128h + 8g .. +8]
};

template <typename E, int D, int TB, bool NT = true>
__device__ __forceinline__ void issue_tile(BTile<D, TB>& T, const E* kbase, const E* vbase,
                                           int64_t block_elems, const int64_t (&phys)[TB],
                                           const bool (&valid)[TB], int g, int grp) {
  constexpr int NH = D / 128;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    if (valid[b]) {
      const E* kb = kbase + phys[b] * block_elems;
      const E* vb = vbase + phys[b] * block_elems;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const E* a = kb + (4 * grp + rr) * D + h * 128 + 8 * g;
          T.k[b][rr][h] = NT ? ld16_stream(a) : ld16(a);
        }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const E* a = vb + (4 * grp + rr) * D + h * 128 + 8 * g;
          T.v[b][rr][h] = NT ? ld16_stream(a) : ld16(a);
        }
    } else {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          T.k[b][rr][h] = (u32x4){0u, 0u, 0u, 0u};
          T.v[b][rr][h] = (u32x4){0u, 0u, 0u, 0u};
        }
    }
  }
}

// Buffer resource over one (block, KV head) of a cache: `bytes` long, 0 for a
// block outside the context. Loads through a zero-length resource return
// zeros without touching memory, so a tile's loads need no branch. `base`
// and `bytes` must be the same in every lane of the wave (a resource lives in
// scalar registers); readfirstlane states that to the compiler, which would
// otherwise loop over the lanes' values.
constexpr uint32_t kBufferWord3 = 0x00020000;  // gfx9: 32-bit data format, raw access
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ua = reinterpret_cast<void*>(lo | (hi << 32));
  return __builtin_amdgcn_make_buffer_rsrc(ua, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           (int)kBufferWord3);
}
constexpr int kAuxNT = 2;  // cache-policy bits of a buffer load: non-temporal

// Same tile as issue_tile, with branch-free loads: a block with valid[b]
// false reads as zeros and costs no memory traffic. Every wave issues the
// same instructions for every tile, which keeps the compiler's wait counts
// exact when several tiles are in flight.
template <typename E, int D, int TB>
__device__ __forceinline__ void issue_tile_rsrc(BTile<D, TB>& T, const E* kbase, const E* vbase,
                                                int64_t block_elems, const int64_t (&phys)[TB],
                                                const bool (&valid)[TB], int g, int grp) {
  constexpr int NH = D / 128;
  constexpr uint32_t kBytes = (uint32_t)(kBS * D * sizeof(E));
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int64_t off = valid[b] ? phys[b] * block_elems : 0;
    const uint32_t n = valid[b] ? kBytes : 0u;
    const __amdgpu_buffer_rsrc_t kr = block_rsrc(kbase + off, n);
    const __amdgpu_buffer_rsrc_t vr = block_rsrc(vbase + off, n);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int byte = (int)((((4 * grp + rr) * D) + h * 128 + 8 * g) * sizeof(E));
        T.k[b][rr][h] = __builtin_amdgcn_raw_buffer_load_b128(kr, byte, 0, kAuxNT);
      }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int byte = (int)((((4 * grp + rr) * D) + h * 128 + 8 * g) * sizeof(E));
        T.v[b][rr][h] = __builtin_amdgcn_raw_buffer_load_b128(vr, byte, 0, kAuxNT);
      }
  }
}

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
  if (sh->dtype != PA_F32 && sh->dtype != PA_BF16 && sh->dtype != PA_F16) return PA_EUNSUPPORTED;
  if (sh->max_blocks_per_seq > (1 << 26)) return PA_EUNSUPPORTED;  // keeps token counts in int32
  if (sh->partition_size != 0 && sh->partition_size != PA_PARTITION_SIZE &&
      sh->partition_size != PA_PARTITION_SIZE_SMALL)
    return PA_EUNSUPPORTED;
  return PA_OK;
}

// Where a kernel goes: the stream, and optionally a pair of events recorded
// at the start and the end of that kernel alone (measurement entry points).
struct Launch {
  hipStream_t stream;
  hipEvent_t start, stop;
};

template <typename K, typename A>
hipError_t launch(K kern, dim3 grid, dim3 block, size_t smem, const Launch& L, const A& arg) {
  if (L.start || L.stop)
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)smem, L.stream, L.start, L.stop, 0, arg);
  else
    hipLaunchKernelGGL(kern, grid, block, smem, L.stream, arg);
  return hipGetLastError();
}

// Launch with `smem` bytes of dynamic LDS. Above the default 64 KB a kernel
// needs its limit raised; that is done once per kernel and device, to the
// most any call of that kernel can ask for, not on every launch.
template <auto kern, typename A>
hipError_t launch_lds(size_t max_smem, dim3 grid, dim3 block, size_t smem, const Launch& L, const A& P) {
  if (smem > 65536) {
    static std::atomic<uint64_t> raised{0};  // bit d: done on device d
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0;
    if (!bit || !(raised.load(std::memory_order_acquire) & bit)) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_smem);
      if (e != hipSuccess) return e;
      raised.fetch_or(bit, std::memory_order_release);
    }
  }
  return launch(kern, grid, block, smem, L, P);
}

// When there is nothing to launch, a timed call still records its events,
// back to back, so the caller's pair always completes and reads ~0.
hipError_t nothing_launched(const Launch& L) {
  if (L.start && hipEventRecord(L.start, L.stream) != hipSuccess) return hipGetLastError();
  if (L.stop && hipEventRecord(L.stop, L.stream) != hipSuccess) return hipGetLastError();
  return hipSuccess;
}

Launch on(void* stream) { return Launch{(hipStream_t)stream, nullptr, nullptr}; }


}  // namespace
