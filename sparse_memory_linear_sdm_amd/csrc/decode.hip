// Fused single-token step: for one (b,h) per 256-thread block, wave 0 forms
// the write selection from (s1, s2), wave 1 the read selection from (q1, q2)
// (product-key top-K, page "Riepilogo Tecnico: Sparse Delta Memory (SDM)",
// "Meccanismo Core" item 2), the other waves stage v; then the whole block
// applies the gated delta write to the W rows (item 3), and after a block
// barrier (which makes the block's stores visible to its own loads) reads
// the R rows and forms o = sum_j r_j M[g_j] (item 4).
#include "internal.h"
#include "select_wave.h"

namespace sdm {
namespace {

constexpr int kDecThreads = 256;

template <int P, bool BF16>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    void* __restrict__ Mv, int64_t N, int n, int d_v, int W, int R, const float* __restrict__ s1,
    const float* __restrict__ s2, const float* __restrict__ q1, const float* __restrict__ q2,
    const float* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ out, int32_t* __restrict__ widx_out, int32_t* __restrict__ ridx_out) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ES;
  __shared__ SelectLds sl[2];
  __shared__ int32_t s_widx[64], s_ridx[64];
  __shared__ float s_wk[64], s_rw[64];
  __shared__ float s_v[256];
  __shared__ float s_red[4096 / ES];

  const int mem = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  if (w == 0) {
    select_unit<P>(s1 + (int64_t)mem * n, s2 + (int64_t)mem * n, n, W, sl[0], s_widx, nullptr,
                   s_wk);
  } else if (w == 1) {
    select_unit<P>(q1 + (int64_t)mem * n, q2 + (int64_t)mem * n, n, R, sl[1], s_ridx, nullptr,
                   s_rw);
  } else {
    for (int c = tid - 2 * kWave; c < d_v; c += kDecThreads - 2 * kWave)
      s_v[c] = v[(int64_t)mem * d_v + c];
  }
  __syncthreads();
  if (widx_out && tid < W) widx_out[(int64_t)mem * W + tid] = s_widx[tid];
  if (ridx_out && tid < R) ridx_out[(int64_t)mem * R + tid] = s_ridx[tid];

  const int CPR = d_v * ES / 16;  // 16-byte chunks per row
  const uint32_t Nu = (uint32_t)N;
  char* const Mb = reinterpret_cast<char*>(Mv) + (int64_t)mem * N * d_v * ES;
  const float a = alpha[mem], b = beta[mem];

  // gated delta write of the W rows
  for (int c = tid; c < W * CPR; c += kDecThreads) {
    const int j = c / CPR, p = c - j * CPR;
    const int32_t row = s_widx[j];
    if ((uint32_t)row >= Nu) continue;
    uint4* ptr = reinterpret_cast<uint4*>(Mb + ((int64_t)row * d_v + p * EPL) * ES);
    uint4 q = *ptr;
    const float g = b * s_wk[j];
    float m[EPL];
    if constexpr (BF16) {
      const uint32_t wq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[2 * i] = __uint_as_float(wq[i] << 16);
        m[2 * i + 1] = __uint_as_float(wq[i] & 0xFFFF0000u);
      }
    } else {
      m[0] = __uint_as_float(q.x);
      m[1] = __uint_as_float(q.y);
      m[2] = __uint_as_float(q.z);
      m[3] = __uint_as_float(q.w);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float mt = a * m[e];
      m[e] = fmaf(g, s_v[p * EPL + e] - mt, mt);
    }
    if constexpr (BF16) {
      uint32_t wq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wq[i] = (uint32_t)f32_to_bf16_rne(m[2 * i]) | ((uint32_t)f32_to_bf16_rne(m[2 * i + 1]) << 16);
      q = make_uint4(wq[0], wq[1], wq[2], wq[3]);
    } else {
      q = make_uint4(__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]),
                     __float_as_uint(m[3]));
    }
    *ptr = q;
  }
  __syncthreads();

  // sparse read of the R rows after the write
  const int RG = kDecThreads / CPR;  // row groups
  const int p = tid % CPR, rg = tid / CPR;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  if (rg < RG) {
    for (int j = rg; j < R; j += RG) {
      const int32_t row = s_ridx[j];
      if ((uint32_t)row >= Nu) continue;
      const uint4 q = *reinterpret_cast<const uint4*>(Mb + ((int64_t)row * d_v + p * EPL) * ES);
      const float r = s_rw[j];
      if constexpr (BF16) {
        const uint32_t wq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(r, __uint_as_float(wq[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(r, __uint_as_float(wq[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
      } else {
        acc[0] = fmaf(r, __uint_as_float(q.x), acc[0]);
        acc[1] = fmaf(r, __uint_as_float(q.y), acc[1]);
        acc[2] = fmaf(r, __uint_as_float(q.z), acc[2]);
        acc[3] = fmaf(r, __uint_as_float(q.w), acc[3]);
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_red[rg * d_v + p * EPL + e] = acc[e];
  }
  __syncthreads();
  for (int c = tid; c < d_v; c += kDecThreads) {
    float sum = 0.0f;
    for (int g2 = 0; g2 < RG; ++g2) sum += s_red[g2 * d_v + c];
    out[(int64_t)mem * d_v + c] = sum;
  }
}

template <int P>
hipError_t launch(void* M, int dtype, int n_mem, int n, int d_v, int W, int R, const float* s1,
                  const float* s2, const float* q1, const float* q2, const float* v,
                  const float* alpha, const float* beta, float* out, int32_t* widx,
                  int32_t* ridx, hipStream_t stream) {
  const int64_t N = (int64_t)n * n;
  if (dtype == 1)
    hipLaunchKernelGGL((decode_kernel<P, true>), dim3(n_mem), dim3(kDecThreads), 0, stream, M, N,
                       n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx);
  else
    hipLaunchKernelGGL((decode_kernel<P, false>), dim3(n_mem), dim3(kDecThreads), 0, stream, M,
                       N, n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_decode(void* M, int dtype, int B, int H, int n, int d_v, int W, int R,
                              const float* s1, const float* s2, const float* q1,
                              const float* q2, const float* v, const float* alpha,
                              const float* beta, float* out, int32_t* widx, int32_t* ridx,
                              hipStream_t stream) {
  const int n_mem = B * H;
  switch (n <= 64 ? 1 : n / 64) {
    case 1: return launch<1>(M, dtype, n_mem, n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx, stream);
    case 2: return launch<2>(M, dtype, n_mem, n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx, stream);
    case 4: return launch<4>(M, dtype, n_mem, n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx, stream);
    case 8: return launch<8>(M, dtype, n_mem, n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx, stream);
    case 16: return launch<16>(M, dtype, n_mem, n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx, stream);
    case 32: return launch<32>(M, dtype, n_mem, n, d_v, W, R, s1, s2, q1, q2, v, alpha, beta, out, widx, ridx, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdm
