// decode_common.h - device helpers shared by the two decode kernels (internal header).
//
// Operand types, MFMA wrappers, device-scope partial stores and loads, and the
// per-lane registers of one 32-token chunk (key rows and value tiles) with the
// logits product over them.  See decode.hip for the operand layouts.
#pragma once

#include <math.h>

#include "kernels.h"

namespace pa {
namespace dec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define AS4 __attribute__((address_space(4)))  // constant address space: scalar loads

constexpr int NW = kWavesPerGroup;
constexpr int NT_THREADS = NW * 64;

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  typedef bf16x8 type;
};
template <>
struct Vec8<_Float16> {
  typedef f16x8 type;
};

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// a 16-byte load of data read once per call (non-temporal: kept out of the way of
// data that is reused)
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// a 16-byte load with the non-temporal hint when NTL
template <bool NTL>
__device__ __forceinline__ u32x4 ld16_as(const void* p) {
  if constexpr (NTL) return ld16_nt(p);
  else return ld16(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// four consecutive outputs, rounded to nearest even
template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    T t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (T)v[e];
    *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, t);
  }
}

// Partial results cross workgroups (and XCDs, whose L2 caches are not coherent with
// each other) inside one launch.  They are written and read with device-scope
// accesses (the sc1 cache policy), which go to the device's coherence point instead
// of a private L2, so no cache-wide write-back or invalidate is needed: a writer waits
// for its stores to complete (vmcnt 0) before a barrier and the arrival count; a
// reader that saw the count complete reads with device-scope loads.  Rows are moved
// as whole 16-byte pieces through buffer instructions, whose base must be
// wave-uniform and whose offset is 32-bit.
__device__ __forceinline__ void st_dev2(float* p, float a, float b) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p),
                     (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (max, sum) pair of one partial
__device__ __forceinline__ void ld_dev2(const float* p, float& a, float& b) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  a = __uint_as_float((uint32_t)v);
  b = __uint_as_float((uint32_t)(v >> 32));
}
// 16-byte device-scope store / load at byte offset `off` (< 2^31) from a wave-uniform base
__device__ __forceinline__ void st_dev16(float* base, int off, f32x4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 16);
}
__device__ __forceinline__ f32x4 ld_dev16(const float* base, int off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}
// every store this wave has issued is complete (and, device-scope, visible device-wide)
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Registers of one 32-token chunk for one lane (column c = lane % 16, quad i = lane / 16).
template <typename T, int D>
struct Chunk {
  static constexpr int E = sizeof(T);
  static constexpr int KL = D * E / 64;  // 16-byte loads per key row: a quarter of the row
  static constexpr int VL = E / 2;       // 16-byte loads per value tile: 8 tokens
  static constexpr int NT = D / 16;      // 16-dimension output tiles
  u32x4 ka[KL];                          // key row of token tau_a(c), MFMA tile a
  u32x4 kb[KL];                          // key row of token tau_a(c) + 4, tile b
  u32x4 v[NT][VL];                       // values of tokens 8i..8i+7, dimension 16n + c
};

// logits tile: acc[r][c] += sum_d K[row r][d] * q[head c][d]
template <typename T, int D>
__device__ __forceinline__ f32x4 qk_tile(const u32x4 (&k)[Chunk<T, D>::KL],
                                         const u32x4 (&q)[Chunk<T, D>::KL]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
    typedef typename Vec8<T>::type V8;
#pragma unroll
    for (int c = 0; c < Chunk<T, D>::KL; ++c)
      acc = mma16(__builtin_bit_cast(V8, k[c]), __builtin_bit_cast(V8, q[c]), acc);
  } else {
    // bit-cast whole vectors: a bit-cast of one vector element is not safe here
#pragma unroll
    for (int c = 0; c < Chunk<T, D>::KL; ++c) {
      const f32x4 kf = __builtin_bit_cast(f32x4, k[c]);
      const f32x4 qv = __builtin_bit_cast(f32x4, q[c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mma4(kf[e], qv[e], acc);
    }
  }
  return acc;
}

// Lanes c, c + 16, c + 32 and c + 48 (the four quads of a wave) hold parts of the same
// head's row: reduce over them with the gfx950 lane-swap instructions (VALU only).
__device__ __forceinline__ float max_over_quads(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_quads(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace dec
}  // namespace pa
