// Row fragments of the state as the scan kernels move them: 16 bytes per
// lane, unpacked to fp32 for the update and packed back to the state type,
// and the gated delta write of one element (page "Riepilogo Tecnico: Sparse
// Delta Memory (SDM)", section "Meccanismo Core", item 3).
#pragma once
#include "device_common.h"

namespace sdm {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

template <typename DT>
__device__ __forceinline__ void unpack(const u32x4v& q, float (&f)[16 / sizeof(DT)]) {
  if constexpr (sizeof(DT) == 1) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  } else if constexpr (sizeof(DT) == 4) {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  } else {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

template <typename DT>
__device__ __forceinline__ u32x4v pack(const float (&f)[16 / sizeof(DT)]) {
  if constexpr (sizeof(DT) == 1) {
    return u32x4v{f32x4_to_fp8x4(f[0], f[1], f[2], f[3]), f32x4_to_fp8x4(f[4], f[5], f[6], f[7]),
                  f32x4_to_fp8x4(f[8], f[9], f[10], f[11]),
                  f32x4_to_fp8x4(f[12], f[13], f[14], f[15])};
  } else if constexpr (sizeof(DT) == 4) {
    return u32x4v{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                  __float_as_uint(f[3])};
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_rne(f[2 * i]) | ((uint32_t)f32_to_bf16_rne(f[2 * i + 1]) << 16);
    return u32x4v{w[0], w[1], w[2], w[3]};
  }
}

__device__ __forceinline__ u32x4v lds_u4(const uint4& x) { return u32x4v{x.x, x.y, x.z, x.w}; }

// The gated delta write of one element.  For fp8 state the stored code is
// decided by this binary32 result, so it is taken in a fixed order with no
// contraction: Mt = alpha*m, d = v - Mt, u = fma(beta*k, d, Mt).
__device__ __forceinline__ float write_elem_exact(float a, float g, float v, float m) {
#pragma clang fp contract(off)
  const float mt = a * m;
  const float d = v - mt;
  return __builtin_fmaf(g, d, mt);
}

// The gated delta write of one element in the state's arithmetic: fp32 with
// a fused multiply-add for fp32 and bf16 state, the fixed binary32 order
// above for fp8 state.
template <typename DT>
__device__ __forceinline__ float write_elem(float a, float g, float v, float m) {
  if constexpr (sizeof(DT) == 1) {
    return write_elem_exact(a, g, v, m);
  } else {
    const float mt = a * m;
    return fmaf(g, v - mt, mt);
  }
}

}  // namespace sdm
