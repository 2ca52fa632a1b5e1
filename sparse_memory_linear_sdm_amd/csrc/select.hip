// Selection kernel: product-key top-K with softmax weights, fully parallel
// over units (one unit = one (b,h,t) key or query), one wavefront per unit.
#include "internal.h"
#include "select_wave.h"

namespace sdm {
namespace {

constexpr int kSelWaves = 4;  // units per 256-thread block

template <int P>
__global__ __launch_bounds__(kSelWaves * kWave) void select_kernel(
    const float* __restrict__ x1, const float* __restrict__ x2, int64_t units, int n, int K,
    int32_t* __restrict__ idx, float* __restrict__ score, float* __restrict__ weight) {
  __shared__ SelectLds lds[kSelWaves];
  const int w = threadIdx.x / kWave;
  const int64_t unit = (int64_t)blockIdx.x * kSelWaves + w;
  if (unit >= units) return;  // whole wave leaves; no block-wide barrier below
  select_unit<P>(x1 + unit * n, x2 + unit * n, n, K, lds[w], idx + unit * K,
                 score ? score + unit * K : nullptr, weight + unit * K);
}

template <int P>
hipError_t launch(const float* x1, const float* x2, int64_t units, int n, int K, int32_t* idx,
                  float* score, float* weight, hipStream_t stream) {
  int64_t blocks = (units + kSelWaves - 1) / kSelWaves;
  hipLaunchKernelGGL(select_kernel<P>, dim3((unsigned)blocks), dim3(kSelWaves * kWave), 0,
                     stream, x1, x2, units, n, K, idx, score, weight);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const float* x1, const float* x2, int64_t units, int n, int K,
                         int32_t* idx, float* score, float* weight, hipStream_t stream) {
  if (units == 0) return hipSuccess;
  switch (n <= 64 ? 1 : n / 64) {
    case 1: return launch<1>(x1, x2, units, n, K, idx, score, weight, stream);
    case 2: return launch<2>(x1, x2, units, n, K, idx, score, weight, stream);
    case 4: return launch<4>(x1, x2, units, n, K, idx, score, weight, stream);
    case 8: return launch<8>(x1, x2, units, n, K, idx, score, weight, stream);
    case 16: return launch<16>(x1, x2, units, n, K, idx, score, weight, stream);
    case 32: return launch<32>(x1, x2, units, n, K, idx, score, weight, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdm
