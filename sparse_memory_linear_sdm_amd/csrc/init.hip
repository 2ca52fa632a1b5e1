// State-init kernel (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)",
// section "Stato Iniziale Appreso": each sequence starts from the learned
// table M0).  M[b,h] = M0[h]; a streaming copy that reads each M0 element
// once and writes it B times (bf16 state: rounded to nearest even).
#include "device_common.h"
#include "internal.h"

namespace sdm {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void init_kernel(void* __restrict__ M,
                                                   const f32x4* __restrict__ M0, int B, int H,
                                                   int64_t per4) {
  const int64_t total = (int64_t)H * per4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const f32x4 f = __builtin_nontemporal_load(M0 + i);
    const int64_t h = i / per4;
    const int64_t r = i - h * per4;
    for (int b = 0; b < B; ++b) {
      const int64_t o = ((int64_t)b * H + h) * per4 + r;
      if constexpr (BF16) {
        u32x2 p;
        p.x = (uint32_t)f32_to_bf16_rne(f.x) | ((uint32_t)f32_to_bf16_rne(f.y) << 16);
        p.y = (uint32_t)f32_to_bf16_rne(f.z) | ((uint32_t)f32_to_bf16_rne(f.w) << 16);
        __builtin_nontemporal_store(p, reinterpret_cast<u32x2*>(M) + o);
      } else {
        __builtin_nontemporal_store(f, reinterpret_cast<f32x4*>(M) + o);
      }
    }
  }
}

}  // namespace

hipError_t launch_state_init(void* M, int dtype, const float* M0, int B, int H, int64_t N,
                             int d_v, hipStream_t stream) {
  const int64_t per4 = N * d_v / 4;
  const int64_t total = (int64_t)H * per4;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (dtype == 1)
    hipLaunchKernelGGL(init_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, M,
                       reinterpret_cast<const f32x4*>(M0), B, H, per4);
  else
    hipLaunchKernelGGL(init_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, M,
                       reinterpret_cast<const f32x4*>(M0), B, H, per4);
  return hipGetLastError();
}

}  // namespace sdm
