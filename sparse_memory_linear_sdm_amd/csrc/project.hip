// Token projections, the step's front end (page "Riepilogo Tecnico: Sparse
// Delta Memory (SDM)", section "Meccanismo Core", item 2: the projected keys
// k' and queries q' are split in two halves; section "Design IsoFLOP": the
// projections are sized like the baseline's).  Per token x (d_model bf16
// values) and head h, y = W_h x (P = 4n + d_v + 2 rows per head: the key
// halves s1, s2, the query halves q1, q2, v, and the two gate
// pre-activations); alpha = sigmoid(y_alpha), beta = sigmoid(y_beta).
//
// This is the one dense contraction of the path, so it runs on the matrix
// cores: C = X * Wt^T, X [M, K] and Wt [Ncols, K] bf16 (both K-contiguous),
// fp32 accumulation with v_mfma_f32_32x32x16_bf16.  Per 256-thread workgroup
// a 128 x 128 tile of C (2 x 2 wavefronts of 64 x 64, each 2 x 2 MFMA blocks
// of 32 x 32); K is consumed 64 at a time through double-buffered LDS tiles
// (rows padded by 16 bytes), the next tiles' global loads in flight while
// the current ones feed the MFMAs.  Tiles are numbered so that each XCD gets
// a contiguous range, grouped 8 tiles deep along M, so the workgroups that
// run together on an XCD share their X rows and W columns in its L2.
//
// The epilogue writes each value straight to where the selection and the
// scan read it: s1, s2, q1, q2 [B, H, T, n], v [B, H, T, d_v], alpha, beta
// [B, H, T] (token m = b*T + t), fp32, so no layout pass follows.
#include "device_common.h"
#include "internal.h"

namespace sdm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPBM = kProjTile, kPBN = kProjTile, kPBK = 64, kPPad = 8;  // tile sizes, bf16 elements
constexpr int kPThreads = 256;
constexpr int kPGroupM = 8;

struct ProjArgs {
  const uint16_t* X;   // [M, K] bf16
  const uint16_t* Wt;  // [Ncols, K] bf16, Ncols = H * P
  int64_t M;
  int K;
  int H, P, n, d_v, T;
  int64_t Ncols;
  float *s1, *s2, *q1, *q2, *v, *alpha, *beta;
  int nbm, nbn;
};

struct ProjShared {
  uint16_t a[2][kPBM][kPBK + kPPad];
  uint16_t b[2][kPBN][kPBK + kPPad];
};

__device__ __forceinline__ float sigmoidf_(float y) { return 1.0f / (1.0f + expf(-y)); }

__global__ __launch_bounds__(kPThreads) void project_kernel(ProjArgs A) {
  __shared__ __align__(16) ProjShared sh;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;

  // tile of this workgroup
  const int64_t nblocks = (int64_t)A.nbm * A.nbn;
  int64_t pid = blockIdx.x;
  if (nblocks % 8 == 0) pid = (pid & 7) * (nblocks / 8) + (pid >> 3);  // a contiguous range per XCD
  const int64_t per_group = (int64_t)kPGroupM * A.nbn;
  const int64_t first_m = (pid / per_group) * kPGroupM;
  const int64_t gsz = (A.nbm - first_m) < kPGroupM ? (A.nbm - first_m) : kPGroupM;
  const int64_t pm = first_m + (pid % per_group) % gsz;
  const int64_t pn = (pid % per_group) / gsz;
  const int64_t m0 = pm * kPBM, n0 = pn * kPBN;

  // global -> LDS: 1024 16-byte segments per operand tile, 4 per thread
  uint4 ra[4], rb[4];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + kPThreads * q, row = c >> 3, seg = c & 7;
      const int64_t gm = m0 + row, gn = n0 + row;
      const bool vm = gm < A.M, vn = gn < A.Ncols;
      const uint4 xa = *reinterpret_cast<const uint4*>(A.X + (vm ? gm : A.M - 1) * A.K + k0 + seg * 8);
      const uint4 xb = *reinterpret_cast<const uint4*>(A.Wt + (vn ? gn : A.Ncols - 1) * A.K + k0 + seg * 8);
      ra[q] = vm ? xa : make_uint4(0, 0, 0, 0);
      rb[q] = vn ? xb : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = tid + kPThreads * q, row = c >> 3, seg = c & 7;
      *reinterpret_cast<uint4*>(&sh.a[buf][row][seg * 8]) = ra[q];
      *reinterpret_cast<uint4*>(&sh.b[buf][row][seg * 8]) = rb[q];
    }
  };

  const int wm = w & 1, wn = w >> 1;  // this wavefront's 64 x 64 quarter of the tile
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = A.K / kPBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kPBK);  // in flight during the MFMAs
#pragma unroll
    for (int kk = 0; kk < kPBK; kk += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&sh.a[buf][wm * 64 + i * 32 + lr][kk + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&sh.b[buf][wn * 64 + j * 32 + lr][kk + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  }

  // epilogue: lane l, accumulator r of block (i, j) holds C[row][col] with
  // row = 8*(r/4) + 4*(l/32) + r%4 and col = l%32 within the 32 x 32 block
  const int64_t HT = (int64_t)A.H * A.T;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t col = n0 + wn * 64 + j * 32 + lr;
    if (col >= A.Ncols) continue;
    const int h = (int)(col / A.P), p = (int)(col % A.P);
    float* dst;
    int64_t stride;  // elements per token of the destination
    int off;
    bool gate = false;
    if (p < 4 * A.n) {
      const int part = p / A.n;
      dst = part == 0 ? A.s1 : part == 1 ? A.s2 : part == 2 ? A.q1 : A.q2;
      stride = A.n;
      off = p - part * A.n;
    } else if (p < 4 * A.n + A.d_v) {
      dst = A.v;
      stride = A.d_v;
      off = p - 4 * A.n;
    } else {
      dst = p == 4 * A.n + A.d_v ? A.alpha : A.beta;
      stride = 1;
      off = 0;
      gate = true;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= A.M) continue;
        const int64_t b = row / A.T, t = row - b * A.T;
        const int64_t tok = b * HT + (int64_t)h * A.T + t;  // ((b*H + h)*T + t)
        const float y = acc[i][j][r];
        dst[tok * stride + off] = gate ? sigmoidf_(y) : y;
      }
    }
  }
}

}  // namespace

hipError_t launch_project(const uint16_t* X, const uint16_t* Wt, int B, int T, int d_model, int H,
                          int n, int d_v, float* s1, float* s2, float* q1, float* q2, float* v,
                          float* alpha, float* beta, hipStream_t stream) {
  ProjArgs A;
  A.X = X;
  A.Wt = Wt;
  A.M = (int64_t)B * T;
  A.K = d_model;
  A.H = H;
  A.P = 4 * n + d_v + 2;
  A.n = n;
  A.d_v = d_v;
  A.T = T;
  A.Ncols = (int64_t)H * A.P;
  A.s1 = s1;
  A.s2 = s2;
  A.q1 = q1;
  A.q2 = q2;
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  if (A.M == 0) return hipSuccess;
  A.nbm = (int)((A.M + kPBM - 1) / kPBM);
  A.nbn = (int)((A.Ncols + kPBN - 1) / kPBN);
  const int64_t blocks = project_blocks(A.M, A.Ncols);
  hipLaunchKernelGGL(project_kernel, dim3((unsigned)blocks), dim3(kPThreads), 0, stream, A);
  return hipGetLastError();
}

}  // namespace sdm
