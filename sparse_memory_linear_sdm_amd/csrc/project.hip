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
// fp32 accumulation with v_mfma_f32_32x32x16_bf16.  Per 512-thread workgroup
// a 256 x 256 tile of C: 2 x 4 wavefronts of 128 x 64, each 4 x 2 MFMA
// blocks of 32 x 32.  K is consumed 64 at a time through two LDS stages
// (128 KiB) filled by direct global-to-LDS loads (no staging registers, no
// LDS store instructions): the loads of stage k+1 are issued right after the
// barrier of stage k and land while stage k feeds the MFMAs; one barrier per
// stage (measured: 64-deep stages, two of them, beat 32-deep ones in a ring
// of 2 to 5 by 10%: half the barriers).  Within a stage each operand row is
// 128 bytes (eight 16-byte segments), and segment s of row r sits at
// position s ^ ((r >> 1) & 7): with that placement the fragment reads (32
// rows x one segment per half-wave) measured free of bank conflicts on
// gfx950, while unswizzled rows conflict.  Tiles are numbered so that each
// XCD gets a contiguous range, grouped 8 tiles deep along M, so the
// workgroups that run together on an XCD share their X rows and W columns in
// its L2.
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

constexpr int kPBM = kProjTile, kPBN = kProjTile;  // output tile
constexpr int kPBK = 64;                            // K per stage (bf16 elements)
constexpr int kPStages = 2;
constexpr int kPThreads = 512;                      // 8 wavefronts
constexpr int kPWavesM = 2;                         // wavefront grid 2 (M) x 4 (N)
constexpr int kPTM = 4, kPTN = 2;                   // 32 x 32 MFMA blocks per wavefront
constexpr int kPSegs = kPBK / 8;                    // 16-byte segments per row
constexpr int kPStage = (kPBM + kPBN) * kPBK;       // bf16 elements per stage
constexpr int kPLoads = kPBM * kPSegs / kPThreads;  // direct loads per thread, operand, stage
constexpr int kPGroupM = 8;
static_assert(kPBM == 256 && kPBN == 256, "the wavefront grid covers 256 x 256");
static_assert(kPLoads == 4 && kPSegs == 8, "the slot numbering assumes 4 loads of 8 segments");

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

__device__ __forceinline__ float sigmoidf_(float y) { return 1.0f / (1.0f + expf(-y)); }

// position of 16-byte segment `seg` in row `row` of a stage
__device__ __forceinline__ int seg_pos(int row, int seg) { return seg ^ ((row >> 1) & 7); }

// s_waitcnt with only the vector-memory count limited (expcnt and lgkmcnt at
// their maxima): vmcnt(n) for n < 16
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8); }

// a workgroup barrier without a memory fence (the direct loads are waited for
// by count just before it); the empty asm keeps the compiler from moving LDS
// accesses across it
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kPThreads) void project_kernel(ProjArgs A) {
  __shared__ __align__(16) uint16_t lds[kPStages * kPStage];
  const int tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);

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

  // Direct loads: per operand and stage, load q of wavefront w fills the 64
  // consecutive 16-byte slots (q * 8 + w) * 64 + lane; slot s is position
  // s % 8 of row s / 8, so it takes segment seg_pos(row, s % 8) of that row.
  // Rows past the matrix read its last row (their products land only in
  // outputs that are never stored).
  const uint16_t* srcA[kPLoads];
  const uint16_t* srcB[kPLoads];
#pragma unroll
  for (int q = 0; q < kPLoads; ++q) {
    const int s = (q * 8 + w) * kWave + lane, row = s / kPSegs, seg = seg_pos(row, s % kPSegs);
    const int64_t gm = m0 + row < A.M ? m0 + row : A.M - 1;
    const int64_t gn = n0 + row < A.Ncols ? n0 + row : A.Ncols - 1;
    srcA[q] = A.X + gm * A.K + seg * 8;
    srcB[q] = A.Wt + gn * A.K + seg * 8;
  }
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    uint16_t* base = lds + buf * kPStage;
#pragma unroll
    for (int q = 0; q < kPLoads; ++q) {
      __builtin_amdgcn_global_load_lds((const void*)(srcA[q] + kt * kPBK),
                                       (void*)(base + (q * 8 + w) * kWave * 8), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(srcB[q] + kt * kPBK),
                                       (void*)(base + kPBM * kPBK + (q * 8 + w) * kWave * 8), 16,
                                       0, 0);
    }
  };

  const int wm = w % kPWavesM, wn = w / kPWavesM;  // this wavefront's 128 x 64 part of the tile
  const int lr = lane & 31, lh = lane >> 5;
  // LDS offsets (elements, within a stage) of this lane's fragments for the
  // first 16 of the stage's 64 k; the k-th 16 are segments 2k, 2k + 1, at
  // offset ^ 16k
  int offA[kPTM], offB[kPTN];
#pragma unroll
  for (int i = 0; i < kPTM; ++i) {
    const int row = (wm * kPTM + i) * 32 + lr;
    offA[i] = row * kPBK + seg_pos(row, lh) * 8;
  }
#pragma unroll
  for (int j = 0; j < kPTN; ++j) {
    const int row = (wn * kPTN + j) * 32 + lr;
    offB[j] = kPBM * kPBK + row * kPBK + seg_pos(row, lh) * 8;
  }
  f32x16 acc[kPTM][kPTN];
#pragma unroll
  for (int i = 0; i < kPTM; ++i)
#pragma unroll
    for (int j = 0; j < kPTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = A.K / kPBK;
#pragma unroll
  for (int s = 0; s < kPStages - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once this wavefront's loads are in (they are the
    // only ones outstanding)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    stage_barrier();  // every wavefront's part of stage kt is in; stage kt-1 is read
    if (kt + kPStages - 1 < nk) issue(kt + kPStages - 1, (kt + kPStages - 1) % kPStages);
    const uint16_t* base = lds + (kt % kPStages) * kPStage;
#pragma unroll
    for (int kk = 0; kk < kPBK / 16; ++kk) {
      bf16x8 a[kPTM], b[kPTN];
#pragma unroll
      for (int i = 0; i < kPTM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(base + (offA[i] ^ (kk * 16)));
#pragma unroll
      for (int j = 0; j < kPTN; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(base + (offB[j] ^ (kk * 16)));
#pragma unroll
      for (int i = 0; i < kPTM; ++i)
#pragma unroll
        for (int j = 0; j < kPTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    // scheduling hint for the stage body: the compiler's single-wavefront
    // small-GEMM strategy, which spreads the fragment reads between the
    // MFMAs (measured 2.5% faster than its default order)
    __builtin_amdgcn_iglp_opt(1);
  }

  // epilogue: lane l, accumulator r of block (i, j) holds C[row][col] with
  // row = 8*(r/4) + 4*(l/32) + r%4 and col = l%32 within the 32 x 32 block
  const int64_t HT = (int64_t)A.H * A.T;
#pragma unroll
  for (int j = 0; j < kPTN; ++j) {
    const int64_t col = n0 + (wn * kPTN + j) * 32 + lr;
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
    for (int i = 0; i < kPTM; ++i) {
      // this lane's rows in block i: rb + 8*(r/4) + r%4, r = 0..15; the
      // token (b, t) of rb by one division (tokens < 2^32), then stepped
      const int64_t rb = m0 + (wm * kPTM + i) * 32 + 4 * lh;
      if (rb >= A.M) continue;
      uint32_t b = (uint32_t)rb / (uint32_t)A.T, t = (uint32_t)rb - b * (uint32_t)A.T;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r > 0) {
          t += (r & 3) ? 1 : 5;  // the row offsets run 0,1,2,3, 8,9,10,11, 16,...
          while (t >= (uint32_t)A.T) {
            t -= (uint32_t)A.T;
            ++b;
          }
        }
        const int64_t row = rb + 8 * (r >> 2) + (r & 3);
        if (row >= A.M) break;
        const int64_t tok = (int64_t)b * HT + (int64_t)h * A.T + t;  // ((b*H + h)*T + t)
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
