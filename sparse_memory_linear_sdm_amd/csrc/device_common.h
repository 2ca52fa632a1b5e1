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

// ---- cross-lane exchange without LDS.  Every helper below assumes that all
// 64 lanes of the wave are active.
//
// lane_xor(v, o) returns the value of lane (lane ^ o) for o in {1,2,4,8,16,32}:
//   o = 1, 2   DPP quad_perm [1,0,3,2] / [2,3,0,1]
//   o = 4      DPP row_ror:12 (lane i reads i+4 in its row of 16) for lanes
//              with bit 2 clear, row_ror:4 (reads i-4) for the others
//   o = 8      DPP row_ror:8 (i+8 mod 16 == i^8 within a row)
//   o = 16     v_permlane16_swap(v, v) yields {value of lane i & ~16, value
//              of lane i | 16}; take the one that is not the lane's own
//   o = 32     v_permlane32_swap likewise with bit 5.
// The o argument must fold to a constant at the call site.
//
// Two forms of each DPP move: dpp_* (an "old" operand of 0) lets the compiler
// fold the move into the DPP source of the arithmetic that consumes it (as
// in the reductions below); dpp_mov<> takes no old operand -- every lane of
// these permutations has a source lane -- so a plain exchange costs no
// register initialisation.
__device__ __forceinline__ uint32_t dpp_qp_xor1(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_qp_xor2(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_ror4(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, 0x124, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_ror8(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_ror12(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, 0x12C, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int o) {
  const int lane = lane_id();
  switch (o) {
    case 1: return dpp_mov<0xB1>(v);
    case 2: return dpp_mov<0x4E>(v);
    case 4: {
      uint32_t up = dpp_mov<0x12C>(v), down = dpp_mov<0x124>(v);
      return (lane & 4) ? down : up;
    }
    case 8: return dpp_mov<0x128>(v);
    case 16: {
      auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16) ? r[0] : r[1];
    }
    default: {
      auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32) ? r[0] : r[1];
    }
  }
}

__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Reduction of an associative, commutative, exact operation (integer sum,
// min, max): quad butterflies, then rotations by 4 and 8 inside each row of
// 16 (every lane then holds its row's total), then the two swaps combine
// rows.  The result is returned as a wave-uniform value.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_exact(uint32_t v, Op op) {
  v = op(v, dpp_qp_xor1(v));
  v = op(v, dpp_qp_xor2(v));
  v = op(v, dpp_row_ror4(v));
  v = op(v, dpp_row_ror8(v));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r[0], r[1]);
  auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = op(q[0], q[1]);
  return uniform_u32(v);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_exact(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_exact(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  return (int)wave_reduce_exact((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Floating-point sum: a pure xor butterfly, so that the two lanes of every
// exchange add the same two operands and all lanes end with the same bits.
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __uint_as_float(lane_xor(__float_as_uint(v), o));
  return __uint_as_float(uniform_u32(__float_as_uint(v)));
}

// Exclusive prefix sum of a per-lane count across the wave: inclusive scans
// inside each row of 16 by DPP row_shr 1, 2, 4, 8 (lanes shifted in from
// outside the row read 0), then each row adds the totals of the rows below.
__device__ __forceinline__ int wave_excl_scan_i32(int v) {
  const int lane = lane_id();
  uint32_t x = (uint32_t)v;
  // bound_ctrl: lanes whose source is outside the row read 0
  x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x114, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x118, 0xF, 0xF, true);
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = lane >> 4;
  x += (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
  return (int)x - v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = lane_xor((uint32_t)v, o);
  uint32_t hi = lane_xor((uint32_t)(v >> 32), o);
  return ((uint64_t)hi << 32) | lo;
}

// Value of lane 0, wave-uniform.
__device__ __forceinline__ float lane0_f32(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
}

// Bitonic sort of one 64-bit key per lane, descending across lanes 0..63.
// A compare-exchange keeps the partner's key y when (y > x) equals "this lane
// keeps the larger key"; on y == x either choice leaves the same key.  One
// 64-bit compare and two selects per key and stage.
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t x) {
  int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = shfl_xor_u64(x, j);
      const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0 || k == 64);
      x = ((y > x) == keep_max) ? y : x;
    }
  }
  return x;
}

// Two independent bitonic sorts (same network as above), interleaved so that
// their exchanges overlap.
__device__ __forceinline__ void wave_sort2_desc_u64(uint64_t& x, uint64_t& z) {
  int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = shfl_xor_u64(x, j);
      const uint64_t w = shfl_xor_u64(z, j);
      const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0 || k == 64);
      x = ((y > x) == keep_max) ? y : x;
      z = ((w > z) == keep_max) ? w : z;
    }
  }
}

// bf16 storage: narrowing rounds to nearest even (widening is a 16-bit shift).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// fp8 E4M3 (OCP "e4m3fn") state element.  The gfx950 conversions round to
// nearest even; the values the write produces stay within +-448, so the
// saturation behaviour of the conversion never matters.
struct fp8e4m3 {
  uint8_t bits;
};

// Four binary32 values -> four E4M3 codes, element i in byte i.
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

}  // namespace sdm
