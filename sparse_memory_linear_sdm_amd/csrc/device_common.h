// Device helpers shared by the SDM kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

constexpr int kWave = 64;

// Native clang vectors (the nontemporal builtins need these, not HIP's
// vector structs).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Order-preserving map binary32 -> uint32: a < b (as floats, -0 == +0)
// exactly when key(a) < key(b).  -0.0 is canonicalised to +0.0 first.
__device__ __forceinline__ uint32_t okey(float x) {
  uint32_t b = __float_as_uint(x);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float okey_inv(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Compiler-level ordering of LDS traffic between lanes of one wave.  A wave
// executes its LDS instructions in order, so a fence at wavefront scope plus
// the wave barrier is enough for cross-lane exchange through LDS.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o);
    v = w < v ? w : v;
  }
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Exclusive prefix sum of a per-lane count across the wave.
__device__ __forceinline__ int wave_excl_scan_i32(int v) {
  int lane = lane_id();
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x - v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
  uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one 64-bit key per lane, descending across lanes 0..63.
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t x) {
  int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t y = shfl_xor_u64(x, j);
      bool lower = (lane & j) == 0;
      bool desc = (lane & k) == 0 || k == 64;
      bool keep_max = (lower == desc);
      x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
    }
  }
  return x;
}

// bf16 storage: widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

}  // namespace sdm
