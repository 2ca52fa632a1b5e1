// Fused single-token step for one (b,h) per 256-thread block (page "Riepilogo
// Tecnico: Sparse Delta Memory (SDM)", "Meccanismo Core" items 2-4):
//   1. each of the four waves runs stage 1 of one half (s1, s2, q1, q2) of the
//      product-key top-K; waves 0 and 1 then finish the write and the read
//      selection (item 2); both stages find their K-th key by the radix
//      search, which has the shorter dependent chain;
//   2. the whole block applies the gated delta write to the W rows (item 3);
//   3. it reads the R rows and forms o = sum_j r_j M[g_j] (item 4).
// When a step's rows fit one batch of loads per thread (the decode workload
// does: W, R <= 64 and rows of up to 512 bytes), the gathers of 2 and 3 are
// issued together, before any store: a read row that this step also writes
// is then taken from a copy of its updated value kept in LDS instead of the
// (older) loaded one, so the read does not wait for a second trip to memory.
// Otherwise 2 runs first and 3 after a block barrier (which makes the block's
// stores visible to its own loads).  Every thread issues all of its row loads
// before using any of them; an invalid row loads row 0 (always inside the
// table) and is masked.
#include "internal.h"
#include "select_wave.h"

namespace sdm {
namespace {

constexpr int kDecThreads = 256;
constexpr int kStage = 2048;  // 16-byte LDS entries for updated rows (32 KiB)

template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4& q, float (&m)[BF16 ? 8 : 4]) {
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
}

template <bool BF16>
__device__ __forceinline__ uint4 pack16(const float (&m)[BF16 ? 8 : 4]) {
  if constexpr (BF16) {
    uint32_t wq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wq[i] = (uint32_t)f32_to_bf16_rne(m[2 * i]) | ((uint32_t)f32_to_bf16_rne(m[2 * i + 1]) << 16);
    return make_uint4(wq[0], wq[1], wq[2], wq[3]);
  } else {
    return make_uint4(__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]),
                      __float_as_uint(m[3]));
  }
}

template <int P, bool BF16>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    void* __restrict__ Mv, int64_t N, int n, int d_v, int W, int R, const float* __restrict__ s1,
    const float* __restrict__ s2, const float* __restrict__ q1, const float* __restrict__ q2,
    const float* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ out, int32_t* __restrict__ widx_out, int32_t* __restrict__ ridx_out) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ES;
  constexpr int kU = BF16 ? 4 : 8;  // 16-byte chunks per thread in flight (one batch at d_v = 128)
  __shared__ SelectLds sl[2];
  __shared__ int32_t s_widx[64], s_ridx[64];
  __shared__ float s_wk[64], s_rw[64];
  __shared__ float s_v[256];
  __shared__ float s_red[4096 / ES];
  __shared__ uint4 s_stage[kStage];  // updated rows by write slot (one-batch path)
  __shared__ int32_t s_match[64];    // read slot -> write slot of the same row, or -1
  __shared__ __align__(16) uint32_t s_hist[4][256];  // stage 1's radix-search histogram, one per wave

  const int mem = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid / kWave;

  // the step's v, alpha and beta are loaded first; their latency hides under
  // the selections
  const float vreg = tid < d_v ? v[(int64_t)mem * d_v + tid] : 0.0f;
  const float a = alpha[mem], b = beta[mem];

  // 1. selections: wave w runs stage 1 of half w into the LDS of its
  // selection and sorts its survivors there (the four halves in parallel)
  uint32_t rc[pairtab::kSlots];
  if (w < 2) pair_slots(w == 0 ? W : R, rc);
  {
    const float* x = w == 0 ? s1 : w == 1 ? s2 : w == 2 ? q1 : q2;
    SelectLds& S = sl[w >> 1];
    uint64_t* const list = (w & 1) ? S.sorted.b : S.sorted.a;
    const int K = w < 2 ? W : R;
    stage1_half<P, true>(x + (int64_t)mem * n, n, K, list, S.trash, s_hist[w]);
    sort_survivors(list, K);
  }
  if (tid < d_v) s_v[tid] = vreg;
  __syncthreads();
  if (w == 0) select_finish<true, true>(n, W, sl[0], rc, s_widx, nullptr, s_wk);
  else if (w == 1) select_finish<true, true>(n, R, sl[1], rc, s_ridx, nullptr, s_rw);
  __syncthreads();
  if (widx_out && tid < W) widx_out[(int64_t)mem * W + tid] = s_widx[tid];
  if (ridx_out && tid < R) ridx_out[(int64_t)mem * R + tid] = s_ridx[tid];

  const int CPR = d_v * ES / 16;  // 16-byte chunks per row
  const uint32_t Nu = (uint32_t)N;
  char* const Mb = reinterpret_cast<char*>(Mv) + (int64_t)mem * N * d_v * ES;

  const int nch = W * CPR;            // 16-byte chunks of the W rows
  const int RG = kDecThreads / CPR;   // read row groups
  const int p = tid % CPR, rg = tid / CPR;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;

  if (nch <= kDecThreads * kU && R <= RG * kU && nch <= kStage) {
    // one batch: issue the write-row and the read-row gathers together
    uint4 qw[kU], qr[kU];
    int64_t offw[kU];
    int jw[kU], pw[kU], jr[kU];
    bool okw[kU], okr[kU];
    float r[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = u * kDecThreads + tid;
      const int j = c / CPR;
      pw[u] = c - j * CPR;
      jw[u] = c < nch ? j : 0;
      const int32_t row = c < nch ? s_widx[j] : -1;
      okw[u] = (uint32_t)row < Nu;
      offw[u] = ((int64_t)(okw[u] ? row : 0) * d_v + pw[u] * EPL) * ES;
      qw[u] = *reinterpret_cast<const uint4*>(Mb + offw[u]);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = rg + u * RG;
      jr[u] = j < R ? j : 0;
      const int32_t row = j < R ? s_ridx[j] : -1;
      okr[u] = (uint32_t)row < Nu;
      r[u] = okr[u] ? s_rw[j] : 0.0f;
      qr[u] = *reinterpret_cast<const uint4*>(Mb + ((int64_t)(okr[u] ? row : 0) * d_v + p * EPL) * ES);
    }
    // while they are in flight: wave w matches read slots 16w .. 16w+15
    // against the write rows (lane i holds write row i, lane jj < 16 read
    // row 16w + jj); registers and ballots only, no LDS round trip per slot
    {
      const int lane = tid % kWave;
      const int32_t wrow = lane < W ? s_widx[lane] : -1;
      const bool wok = (uint32_t)wrow < Nu;
      const int jl = w * 16 + (lane & 15);
      const int32_t rrow = jl < R ? s_ridx[jl] : -1;
      int mine = -1;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int32_t row = __builtin_amdgcn_readlane(rrow, jj);
        const uint64_t hit = __ballot(wok && wrow == row);
        const int i = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
        mine = lane == jj ? i : mine;
      }
      if (lane < 16) s_match[jl] = (uint32_t)rrow < Nu ? mine : -1;
    }
    // gated delta write; the updated rows are also kept in LDS
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (!okw[u]) continue;
      float m[EPL];
      unpack16<BF16>(qw[u], m);
      const float g = b * s_wk[jw[u]];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float mt = a * m[e];
        m[e] = fmaf(g, s_v[pw[u] * EPL + e] - mt, mt);
      }
      const uint4 q = pack16<BF16>(m);
      *reinterpret_cast<uint4*>(Mb + offw[u]) = q;
      s_stage[jw[u] * CPR + pw[u]] = q;
    }
    __syncthreads();
    // sparse read: rows written by this step come from LDS
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = okr[u] ? s_match[jr[u]] : -1;
      // read the LDS copy unconditionally and select values (selecting between
      // the two addresses would put qr in scratch memory)
      const uint4 st = s_stage[(i >= 0 ? i : 0) * CPR + p];
      const uint4 q = make_uint4(i >= 0 ? st.x : qr[u].x, i >= 0 ? st.y : qr[u].y,
                                 i >= 0 ? st.z : qr[u].z, i >= 0 ? st.w : qr[u].w);
      float m[EPL];
      unpack16<BF16>(q, m);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = okr[u] ? fmaf(r[u], m[e], acc[e]) : acc[e];
    }
  } else {
    // 2. gated delta write of the W rows
    for (int c0 = 0; c0 < nch; c0 += kDecThreads * kU) {
      uint4 q[kU];
      int64_t off[kU];
      int jj[kU], pp[kU];
      bool ok[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = c0 + u * kDecThreads + tid;
        const int j = c / CPR;
        pp[u] = c - j * CPR;
        jj[u] = c < nch ? j : 0;
        const int32_t row = c < nch ? s_widx[j] : -1;
        ok[u] = (uint32_t)row < Nu;
        off[u] = ((int64_t)(ok[u] ? row : 0) * d_v + pp[u] * EPL) * ES;
        q[u] = *reinterpret_cast<const uint4*>(Mb + off[u]);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (!ok[u]) continue;
        float m[EPL];
        unpack16<BF16>(q[u], m);
        const float g = b * s_wk[jj[u]];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float mt = a * m[e];
          m[e] = fmaf(g, s_v[pp[u] * EPL + e] - mt, mt);
        }
        *reinterpret_cast<uint4*>(Mb + off[u]) = pack16<BF16>(m);
      }
    }
    __syncthreads();

    // 3. sparse read of the R rows after the write
    for (int j0 = rg; j0 < R; j0 += RG * kU) {
      uint4 q[kU];
      float r[kU];
      bool ok[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int j = j0 + u * RG;
        const int32_t row = j < R ? s_ridx[j] : -1;
        ok[u] = (uint32_t)row < Nu;
        r[u] = ok[u] ? s_rw[j] : 0.0f;
        q[u] = *reinterpret_cast<const uint4*>(Mb + ((int64_t)(ok[u] ? row : 0) * d_v + p * EPL) * ES);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float m[EPL];
        unpack16<BF16>(q[u], m);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = ok[u] ? fmaf(r[u], m[e], acc[e]) : acc[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_red[rg * d_v + p * EPL + e] = acc[e];
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
