// State-init kernel (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)",
// section "Stato Iniziale Appreso": each sequence starts from the learned
// table M0).  M[b,h] = M0[h]; a streaming copy that reads each M0 element
// once and writes it B times (bf16 state: rounded to nearest even).
#include "device_common.h"
#include "internal.h"

namespace sdm {
namespace {

// Each thread moves kU 16-byte groups of M0 (a block covers kU * 256
// consecutive groups, so every load and store instruction is coalesced),
// then writes them to the B sequences' tables.
constexpr int kU = 4;

template <bool BF16>
__global__ __launch_bounds__(256) void init_kernel(void* __restrict__ M,
                                                   const f32x4* __restrict__ M0, int B, int H,
                                                   int64_t per4) {
  const int64_t total = (int64_t)H * per4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kU;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x * kU + threadIdx.x; i0 < total;
       i0 += stride) {
    f32x4 f[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + (int64_t)u * 256;
      f[u] = i < total ? __builtin_nontemporal_load(M0 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int b = 0; b < B; ++b) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + (int64_t)u * 256;
        if (i >= total) continue;
        const int64_t h = i / per4;
        const int64_t o = ((int64_t)b * H + h) * per4 + (i - h * per4);
        if constexpr (BF16) {
          u32x2 p;
          p.x = (uint32_t)f32_to_bf16_rne(f[u].x) | ((uint32_t)f32_to_bf16_rne(f[u].y) << 16);
          p.y = (uint32_t)f32_to_bf16_rne(f[u].z) | ((uint32_t)f32_to_bf16_rne(f[u].w) << 16);
          reinterpret_cast<u32x2*>(M)[o] = p;
        } else {
          reinterpret_cast<f32x4*>(M)[o] = f[u];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_state_init(void* M, int dtype, const float* M0, int B, int H, int64_t N,
                             int d_v, hipStream_t stream) {
  const int64_t per4 = N * d_v / 4;
  const int64_t total = (int64_t)H * per4;
  int64_t blocks = (total + 256 * kU - 1) / (256 * kU);
  if (blocks > 256 * 4) blocks = 256 * 4;  // 4 blocks per CU keep HBM busy and leave room for concurrent work
  if (dtype == 1)
    hipLaunchKernelGGL(init_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, M,
                       reinterpret_cast<const f32x4*>(M0), B, H, per4);
  else
    hipLaunchKernelGGL(init_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, M,
                       reinterpret_cast<const f32x4*>(M0), B, H, per4);
  return hipGetLastError();
}

}  // namespace sdm
