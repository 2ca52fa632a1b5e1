// State-init kernel (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)",
// section "Stato Iniziale Appreso": each sequence starts from the learned
// table M0).  M[b,h] = M0[h]; a streaming copy that reads each M0 element
// once and writes it B times (bf16 and fp8 E4M3 state: rounded to nearest
// even).
#include "device_common.h"
#include "internal.h"

namespace sdm {
namespace {

// Each thread moves kU groups of 4 (fp32), 8 (bf16) or 16 (fp8) consecutive values of
// M0 -- one 16-byte store per group and sequence -- with a block covering
// kU * 256 consecutive groups, so every load and store is coalesced.  M0 is
// [H, N*d_v] and M is [B, H, N*d_v], so group i of M0 lands at group
// b * (H * groups per head) + i of M: no per-element index arithmetic.
// One group per thread over a grid that covers the whole table once (about
// a million blocks at the mid size) was measured fastest: 7.26 ms alone
// against 7.43 ms with two groups per thread and 7.56-7.84 ms for grids of
// 1-4 resident blocks per compute unit looping over 4-16 groups per thread,
// and the selections that run beside it finish sooner (3.3 against 8.6 ms).
constexpr int kU = 1;

template <int DTYPE>  // 0 fp32, 1 bf16, 2 fp8
__global__ __launch_bounds__(256) void init_kernel(void* __restrict__ M,
                                                   const f32x4* __restrict__ M0, int B, int H,
                                                   int64_t per4) {
  constexpr int G = DTYPE == 2 ? 4 : (DTYPE == 1 ? 2 : 1);  // float4 loads per group
  const int64_t total = (int64_t)H * (per4 / G);  // groups of M0
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kU;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x * kU + threadIdx.x; i0 < total;
       i0 += stride) {
    f32x4 f[kU][G];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + (int64_t)u * 256;
#pragma unroll
      for (int g = 0; g < G; ++g)
        // fp32: one 16-byte load per group, streamed past the caches.  bf16
        // and fp8: G loads of one 64- or 32-byte group that share cache
        // lines, so they are plain loads -- streamed, each went to memory on
        // its own (fp8: 6.05 GB read for 4.29 GB of M0, 2.92 -> 2.48 ms at mid).
        if constexpr (G == 1)
          f[u][g] = i < total ? __builtin_nontemporal_load(M0 + i * G + g)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
        else
          f[u][g] = i < total ? M0[i * G + g] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int b = 0; b < B; ++b) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + (int64_t)u * 256;
        if (i >= total) continue;
        const int64_t o = (int64_t)b * total + i;
        if constexpr (DTYPE == 2) {
          u32x4 p;
          p.x = f32x4_to_fp8x4(f[u][0].x, f[u][0].y, f[u][0].z, f[u][0].w);
          p.y = f32x4_to_fp8x4(f[u][1].x, f[u][1].y, f[u][1].z, f[u][1].w);
          p.z = f32x4_to_fp8x4(f[u][2].x, f[u][2].y, f[u][2].z, f[u][2].w);
          p.w = f32x4_to_fp8x4(f[u][3].x, f[u][3].y, f[u][3].z, f[u][3].w);
          reinterpret_cast<u32x4*>(M)[o] = p;
        } else if constexpr (DTYPE == 1) {
          u32x4 p;
          p.x = (uint32_t)f32_to_bf16_rne(f[u][0].x) | ((uint32_t)f32_to_bf16_rne(f[u][0].y) << 16);
          p.y = (uint32_t)f32_to_bf16_rne(f[u][0].z) | ((uint32_t)f32_to_bf16_rne(f[u][0].w) << 16);
          p.z = (uint32_t)f32_to_bf16_rne(f[u][1].x) | ((uint32_t)f32_to_bf16_rne(f[u][1].y) << 16);
          p.w = (uint32_t)f32_to_bf16_rne(f[u][1].z) | ((uint32_t)f32_to_bf16_rne(f[u][1].w) << 16);
          reinterpret_cast<u32x4*>(M)[o] = p;
        } else {
          reinterpret_cast<f32x4*>(M)[o] = f[u][0];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_state_init(void* M, int dtype, const float* M0, int B, int H, int64_t N,
                             int d_v, hipStream_t stream) {
  const int64_t per4 = N * d_v / 4;
  const int64_t total = (int64_t)H * per4 / (dtype == 2 ? 4 : (dtype == 1 ? 2 : 1));
  int64_t blocks = (total + 256 * kU - 1) / (256 * kU);
  if (blocks > kMaxStrideBlocks) blocks = kMaxStrideBlocks;  // the loop strides over the rest
  if (dtype == 2)
    hipLaunchKernelGGL(init_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, M,
                       reinterpret_cast<const f32x4*>(M0), B, H, per4);
  else if (dtype == 1)
    hipLaunchKernelGGL(init_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, M,
                       reinterpret_cast<const f32x4*>(M0), B, H, per4);
  else
    hipLaunchKernelGGL(init_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, M,
                       reinterpret_cast<const f32x4*>(M0), B, H, per4);
  return hipGetLastError();
}

}  // namespace sdm
