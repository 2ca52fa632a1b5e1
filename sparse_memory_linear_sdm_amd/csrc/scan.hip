// Scan kernel: T sequential steps of the gated delta write and the sparse
// read (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)", section
// "Meccanismo Core", items 3 and 4) for every (b,h) memory.
//
// Layout and parallelism.  The update is independent per column, so each
// memory's d_v columns are split into tiles of 128 bytes (one cache line of a
// slot row); one workgroup owns one (b,h,tile) and walks t = 0..T-1.  Blocks
// are numbered so that all tiles of one memory land on the same XCD (blocks
// are dealt to the 8 XCDs round-robin), so a memory's index, weight and value
// traffic is fetched into one L2.  Nothing here is a dense contraction, so
// there is no MFMA: the kernel is bound by HBM traffic, (2W + R) tile rows
// per step per tile.
//
// Two wavefronts per workgroup:
//   producer  stages each step's metadata (row indices, weights, the tile's
//             v columns, alpha, beta) into an LDS "plan", two chunks of kChunk
//             steps ahead of the consumer (triple buffer), and resolves all
//             read-after-write hazards there: for every row of step u it finds
//             the newest step s in [u - D, u] (s < u for write rows) that
//             writes the same row.  Each step's write set is recorded as a
//             bitmap of hashed rows in LDS; a row whose bit is clear in every
//             window bitmap has no hazard (one LDS read per row and window
//             step, no per-lane loops).  The rare rows whose bit is set are
//             resolved exactly, one wave-uniform ballot per candidate against
//             the write rows of the window steps kept in registers.  Only
//             indices are involved, so this runs ahead of the data.
//   consumer  keeps the row gathers of D steps in flight in a register ring:
//             at step u it issues the 16-byte loads of step u + D, then
//             updates step u's W rows (Mt = alpha*M; M = Mt + (beta*k)(v - Mt)
//             in fp32, rounded to the state type), stores them, keeps them in
//             an LDS ring of the last D + 1 steps, and forms o_u from the R
//             read rows.  A row that the plan marks as written inside the
//             window is taken from that LDS ring instead of the (possibly
//             stale) loaded value.  Loads of step u + D are issued after the
//             stores of every step before u by the same wavefront, so the
//             only rows they can miss are those written in [u, u + D - 1] --
//             exactly the window the producer checks.
// The two waves meet at one workgroup barrier per chunk.
#include "device_common.h"
#include "internal.h"

namespace sdm {
namespace {

constexpr int kChunk = 8;    // steps per plan chunk
constexpr int kNBuf = 3;     // plan chunks resident (consumer: c, c+1; producer: c+2)
constexpr int kBmBits = 14;  // bits of a step's write-set bitmap index (2 KiB per step)
constexpr int kBmWords = (1 << kBmBits) / 32;
constexpr uint32_t kInvalid = 0x80000000u;
constexpr int kRowBits = 22;  // row index bits in plan entries (N <= 2^22)
constexpr uint32_t kRowMask = (1u << kRowBits) - 1;

template <typename DT, int COLS>
struct Tile {
  static constexpr int ES = sizeof(DT);
  static constexpr int TB = COLS * ES;     // tile bytes (<= 128)
  static constexpr int EPL = 16 / ES;      // elements per lane per 16-byte access
  static constexpr int LPR = TB / 16;      // lanes per row
  static constexpr int RPI = kWave / LPR;  // rows per wave instruction
  static constexpr int NI = 64 / RPI;      // instructions for 64 rows
};

// Per-step plan.  Row entries are stored transposed: entry [lr][k] is row
// slot j = k * RPI + lr, so a lane reads its NI rows contiguously.  A row entry
// is the row index | (forward code << 22), or kInvalid.  Forward code 0 means
// "use the loaded value"; otherwise code - 1 = ring * 64 + j' names the
// updated row j' of the step held in LDS ring slot `ring`.
template <int COLS>
struct StepPlan {
  uint32_t wrow[64];
  uint32_t rrow[64];
  float wk[64];
  float rw[64];
  float v[COLS];
  float a, b;
  float pad[2];
};

__device__ __forceinline__ uint32_t row_hash(uint32_t row) {
  return (row * 2654435761u) >> (32 - kBmBits);
}

template <typename DT>
__device__ __forceinline__ void unpack(const uint4& q, float (&f)[16 / sizeof(DT)]) {
  if constexpr (sizeof(DT) == 4) {
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
__device__ __forceinline__ uint4 pack(const float (&f)[16 / sizeof(DT)]) {
  if constexpr (sizeof(DT) == 4) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_rne(f[2 * i]) | ((uint32_t)f32_to_bf16_rne(f[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <typename DT, int COLS, int D>
struct ScanShared {
  using TL = Tile<DT, COLS>;
  StepPlan<COLS> plan[kNBuf][kChunk];
  uint4 upd[D + 1][64 * TL::LPR];  // updated rows of the last D + 1 steps, as stored
  uint32_t bm[D + 1][kBmWords];    // producer: write-set bitmaps of the last D + 1 steps
};

// Producer state carried from chunk to chunk: lane j's write row of step
// u - a in prev[a - 1] (-1 when that slot wrote nothing valid).
template <int D>
struct ProducerRing {
  int32_t prev[D];
};

struct ScanArgs {
  int n_mem;
  int64_t N;
  int d_v;
  int64_t T;
  int W, R;
  const int32_t* widx;
  const float* wk;
  const int32_t* ridx;
  const float* rw;
  const float* v;
  const float* alpha;
  const float* beta;
  float* out;
  int ntiles;
};

// ---------------------------------------------------------------- producer

template <typename DT, int COLS, int D>
__device__ __forceinline__ void produce_chunk(ScanShared<DT, COLS, D>& sh, ProducerRing<D>& ring,
                                              const ScanArgs A, int mem, int tile, int64_t c) {
  using TL = Tile<DT, COLS>;
  const int lane = lane_id();
  const int64_t t0 = c * kChunk;
  if (t0 >= A.T) return;
  const int steps = (int)((A.T - t0) < kChunk ? (A.T - t0) : kChunk);
  StepPlan<COLS>* P = sh.plan[c % kNBuf];
  const int64_t base = (int64_t)mem * A.T + t0;
  const uint32_t Nu = (uint32_t)A.N;
  // Issue all of the chunk's metadata loads first, then consume them.
  int32_t wi[kChunk], ri[kChunk];
  float wkv[kChunk], rwv[kChunk], vv[kChunk], ab[kChunk];
#pragma unroll
  for (int s = 0; s < kChunk; ++s) {
    wi[s] = -1;
    ri[s] = -1;
    wkv[s] = 0.f;
    rwv[s] = 0.f;
    vv[s] = 0.f;
    ab[s] = 0.f;
    if (s < steps) {
      const int64_t t = base + s;
      if (lane < A.W) {
        wi[s] = A.widx[t * A.W + lane];
        wkv[s] = A.wk[t * A.W + lane];
      }
      if (lane < A.R) {
        ri[s] = A.ridx[t * A.R + lane];
        rwv[s] = A.rw[t * A.R + lane];
      }
      if (lane < COLS) vv[s] = A.v[t * A.d_v + (int64_t)tile * COLS + lane];
      if (lane == 0) ab[s] = A.alpha[t];
      if (lane == 1) ab[s] = A.beta[t];
    }
  }
  const int lr = lane % TL::RPI, k = lane / TL::RPI;
  const int tslot = lr * TL::NI + k;  // transposed position of row slot j = lane
#pragma unroll
  for (int s = 0; s < kChunk; ++s) {
    if (s >= steps) break;
    const int64_t u = t0 + s;
    const int cur = (int)(u % (D + 1));
    const bool wvalid = lane < A.W && (uint32_t)wi[s] < Nu;
    const bool rvalid = lane < A.R && (uint32_t)ri[s] < Nu;
    const int32_t wrow = wvalid ? wi[s] : -1;
    const uint32_t hw = row_hash((uint32_t)wi[s]), hr = row_hash((uint32_t)ri[s]);
    // write rows: window steps u-1 .. u-D (bitmaps read before this step's
    // bitmap slot, which held step u-D-1, is recycled)
    bool wcand = false;
#pragma unroll
    for (int a = 1; a <= D; ++a) {
      const int sl = (int)((u - a + (D + 1)) % (D + 1));
      const uint32_t word = sh.bm[sl][hw >> 5];
      wcand |= (u - a >= 0) && ((word >> (hw & 31)) & 1u);
    }
    wcand = wcand && wvalid;
    uint4* clr = reinterpret_cast<uint4*>(sh.bm[cur]);
#pragma unroll
    for (int i = lane; i < kBmWords / 4; i += kWave) clr[i] = make_uint4(0, 0, 0, 0);
    wave_sync();
    if (wvalid) atomicOr(&sh.bm[cur][hw >> 5], 1u << (hw & 31));
    wave_sync();
    // read rows: window steps u .. u-D
    bool rcand = false;
#pragma unroll
    for (int a = 0; a <= D; ++a) {
      const int sl = (int)((u - a + (D + 1)) % (D + 1));
      const uint32_t word = sh.bm[sl][hr >> 5];
      rcand |= (u - a >= 0) && ((word >> (hr & 31)) & 1u);
    }
    rcand = rcand && rvalid;
    // exact resolution of the candidates, newest writer first
    uint32_t wcode = 0, rcode = 0;
    for (uint64_t m = __ballot(wcand); m; m &= m - 1) {
      const int L = __ffsll((unsigned long long)m) - 1;
      const int32_t row = __builtin_amdgcn_readlane(wi[s], L);
      uint32_t code = 0;
#pragma unroll
      for (int a = 1; a <= D; ++a) {
        const uint64_t hit = __ballot(ring.prev[a - 1] == row);
        if (hit) {
          code = 1 + (uint32_t)((u - a) % (D + 1)) * 64 + (uint32_t)(__ffsll((unsigned long long)hit) - 1);
          break;
        }
      }
      if (lane == L) wcode = code;
    }
    for (uint64_t m = __ballot(rcand); m; m &= m - 1) {
      const int L = __ffsll((unsigned long long)m) - 1;
      const int32_t row = __builtin_amdgcn_readlane(ri[s], L);
      uint32_t code = 0;
      const uint64_t hit0 = __ballot(wrow == row);
      if (hit0) {
        code = 1 + (uint32_t)cur * 64 + (uint32_t)(__ffsll((unsigned long long)hit0) - 1);
      } else {
#pragma unroll
        for (int a = 1; a <= D; ++a) {
          const uint64_t hit = __ballot(ring.prev[a - 1] == row);
          if (hit) {
            code = 1 + (uint32_t)((u - a) % (D + 1)) * 64 + (uint32_t)(__ffsll((unsigned long long)hit) - 1);
            break;
          }
        }
      }
      if (lane == L) rcode = code;
    }
#pragma unroll
    for (int a = D - 1; a > 0; --a) ring.prev[a] = ring.prev[a - 1];
    ring.prev[0] = wrow;
    StepPlan<COLS>& p = P[s];
    p.wrow[tslot] = wvalid ? ((uint32_t)wi[s] | (wcode << kRowBits)) : kInvalid;
    p.rrow[tslot] = rvalid ? ((uint32_t)ri[s] | (rcode << kRowBits)) : kInvalid;
    p.wk[tslot] = wkv[s];
    p.rw[tslot] = rwv[s];
    if (lane < COLS) p.v[lane] = vv[s];
    if (lane == 0) p.a = ab[s];
    if (lane == 1) p.b = ab[s];
  }
}

// ---------------------------------------------------------------- consumer

// Buffer descriptor word 3 for raw (untyped) buffer access on gfx9-family GPUs.
constexpr int kBufWord3 = 0x00020000;
// Byte offset that is outside every buffer range the kernel builds (memory
// slices are at most 2^31 bytes): loads there return zero and stores are
// dropped, so invalid rows need no branch around their memory operations.
constexpr uint32_t kOffNone = 0x80000000u;

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

template <typename DT, int COLS, int D>
struct Consumer {
  using TL = Tile<DT, COLS>;
  static constexpr int NI = TL::NI, EPL = TL::EPL, LPR = TL::LPR, RPI = TL::RPI;

  u32x4v wv[D + 1][NI];
  u32x4v rv[D + 1][NI];
  __amdgpu_buffer_rsrc_t mres;  // this memory's tile column, range = the memory slice
  uint32_t row_bytes;            // d_v * sizeof(DT)
  uint32_t lane_off;             // lc * 16

  __device__ __forceinline__ const StepPlan<COLS>& plan(ScanShared<DT, COLS, D>& sh,
                                                        int64_t u) const {
    return sh.plan[(u / kChunk) % kNBuf][u % kChunk];
  }

  __device__ __forceinline__ uint32_t offset_of(uint32_t entry) const {
    return (entry & kInvalid) ? kOffNone : (entry & kRowMask) * row_bytes + lane_off;
  }

  // Gathers of step u (all rows invalid when u is past the end).
  template <int SLOT>
  __device__ __forceinline__ void issue(ScanShared<DT, COLS, D>& sh, int lr, int64_t u,
                                        int64_t T) {
    const StepPlan<COLS>& p = plan(sh, u);
    const bool live = u < T;
    uint32_t wo[NI], ro[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      wo[k] = live ? offset_of(p.wrow[lr * NI + k]) : kOffNone;
      ro[k] = live ? offset_of(p.rrow[lr * NI + k]) : kOffNone;
    }
#pragma unroll
    for (int k = 0; k < NI; ++k) wv[SLOT][k] = __builtin_amdgcn_raw_buffer_load_b128(mres, wo[k], 0, 0);
#pragma unroll
    for (int k = 0; k < NI; ++k) rv[SLOT][k] = __builtin_amdgcn_raw_buffer_load_b128(mres, ro[k], 0, 0);
  }

  template <int SLOT>
  __device__ __forceinline__ void step(ScanShared<DT, COLS, D>& sh, float* out_mem, int d_v,
                                       int64_t T, int64_t col0, int lr, int lc, int64_t u) {
    issue<(SLOT + D) % (D + 1)>(sh, lr, u + D, T);
    const StepPlan<COLS>& p = plan(sh, u);
    uint32_t wr[NI], rr[NI];
    float wkk[NI], rwk[NI], vv[EPL];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      wr[k] = p.wrow[lr * NI + k];
      rr[k] = p.rrow[lr * NI + k];
      wkk[k] = p.wk[lr * NI + k];
      rwk[k] = p.rw[lr * NI + k];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) vv[e] = p.v[lc * EPL + e];
    const float a = p.a, b = p.b;
    uint4* const upd = sh.upd[SLOT];
    // gated delta write
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const uint32_t code = (wr[k] >> kRowBits) & 0x1FFu;
      u32x4v q = wv[SLOT][k];
      if (code && !(wr[k] & kInvalid)) {
        const uint4 f = sh.upd[(code - 1) >> 6][((code - 1) & 63) * LPR + lc];
        q = u32x4v{f.x, f.y, f.z, f.w};
      }
      float m[EPL];
      unpack<DT>(make_uint4(q.x, q.y, q.z, q.w), m);
      const float g = b * wkk[k];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float mt = a * m[e];
        m[e] = fmaf(g, vv[e] - mt, mt);
      }
      const uint4 st = pack<DT>(m);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4v{st.x, st.y, st.z, st.w}, mres,
                                             offset_of(wr[k]), 0, 0);
      upd[(k * RPI + lr) * LPR + lc] = st;
    }
    wave_sync();
    // sparse read of the rows as stored after the write
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const uint32_t code = (rr[k] >> kRowBits) & 0x1FFu;
      u32x4v q = rv[SLOT][k];
      if (code && !(rr[k] & kInvalid)) {
        const uint4 f = sh.upd[(code - 1) >> 6][((code - 1) & 63) * LPR + lc];
        q = u32x4v{f.x, f.y, f.z, f.w};
      }
      float m[EPL];
      unpack<DT>(make_uint4(q.x, q.y, q.z, q.w), m);
      const float r = (rr[k] & kInvalid) ? 0.0f : rwk[k];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(r, m[e], acc[e]);
    }
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], o);
    }
    if (lr == 0) {
      float* o = out_mem + u * d_v + col0;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(o + e) = make_float4(acc[e], acc[e + 1], acc[e + 2],
                                                        acc[e + 3]);
    }
    // end of a plan chunk (the last one may be partial): meet the producer,
    // which passes one barrier per chunk
    if ((u % kChunk) == kChunk - 1 || u == T - 1) __syncthreads();
  }
};

template <typename DT, int COLS, int D>
__global__ __launch_bounds__(2 * kWave) void scan_kernel(DT* __restrict__ M, ScanArgs A) {
  using TL = Tile<DT, COLS>;
  __shared__ ScanShared<DT, COLS, D> sh;

  // XCD-aware numbering: bid = ((g * ntiles) + tile) * 8 + x, memory = g*8 + x.
  const int bid = blockIdx.x;
  const int x = bid & 7;
  const int rest = bid >> 3;
  const int tile = rest % A.ntiles;
  const int mem = (rest / A.ntiles) * 8 + x;
  if (mem >= A.n_mem) return;  // whole workgroup leaves together

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t T = A.T;
  const int64_t nchunks = (T + kChunk - 1) / kChunk;

  if (wave == 1) {
    // producer
    ProducerRing<D> ring;
#pragma unroll
    for (int a = 0; a < D; ++a) ring.prev[a] = -1;
    produce_chunk<DT, COLS, D>(sh, ring, A, mem, tile, 0);
    produce_chunk<DT, COLS, D>(sh, ring, A, mem, tile, 1);
    __syncthreads();
    for (int64_t c = 0; c < nchunks; ++c) {
      produce_chunk<DT, COLS, D>(sh, ring, A, mem, tile, c + 2);
      __syncthreads();
    }
    return;
  }

  // consumer
  const int lr = lane / TL::LPR;
  const int lc = lane % TL::LPR;
  const int d_v = A.d_v;
  const int64_t col0 = (int64_t)tile * COLS + lc * TL::EPL;
  DT* const Mm = M + (int64_t)mem * A.N * d_v;
  float* const out_mem = A.out + (int64_t)mem * T * d_v;
  Consumer<DT, COLS, D> cs;
  cs.row_bytes = (uint32_t)(d_v * sizeof(DT));
  cs.lane_off = (uint32_t)(lc * 16);
  cs.mres = __builtin_amdgcn_make_buffer_rsrc(
      Mm + (int64_t)tile * COLS, 0,
      (int)(A.N * d_v * (int64_t)sizeof(DT) - (int64_t)tile * COLS * (int64_t)sizeof(DT)),
      kBufWord3);
  __syncthreads();
  // prologue: gathers of steps 0 .. D-1
  cs.template issue<0>(sh, lr, 0, T);
  if constexpr (D >= 2) cs.template issue<1>(sh, lr, 1, T);
  if constexpr (D >= 3) cs.template issue<2>(sh, lr, 2, T);
  int64_t u = 0;
  for (; u + D + 1 <= T; u += D + 1) {
    cs.template step<0>(sh, out_mem, d_v, T, col0, lr, lc, u);
    cs.template step<1 % (D + 1)>(sh, out_mem, d_v, T, col0, lr, lc, u + 1);
    if constexpr (D >= 2) cs.template step<2 % (D + 1)>(sh, out_mem, d_v, T, col0, lr, lc, u + 2);
    if constexpr (D >= 3) cs.template step<3 % (D + 1)>(sh, out_mem, d_v, T, col0, lr, lc, u + 3);
  }
  // tail: fewer than D + 1 steps
  if (u < T) cs.template step<0>(sh, out_mem, d_v, T, col0, lr, lc, u);
  if (u + 1 < T) cs.template step<1 % (D + 1)>(sh, out_mem, d_v, T, col0, lr, lc, u + 1);
  if constexpr (D >= 3) {
    if (u + 2 < T) cs.template step<2 % (D + 1)>(sh, out_mem, d_v, T, col0, lr, lc, u + 2);
  }
}

template <typename DT, int COLS>
hipError_t launch(void* M, const ScanArgs& A, hipStream_t stream) {
  constexpr int D = 2;
  static_assert(D >= 1 && D <= 3 && D <= kChunk, "prefetch depth");
  const int groups = (A.n_mem + 7) / 8;
  const int64_t blocks = (int64_t)groups * A.ntiles * 8;
  hipLaunchKernelGGL((scan_kernel<DT, COLS, D>), dim3((unsigned)blocks), dim3(2 * kWave), 0,
                     stream, reinterpret_cast<DT*>(M), A);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(void* M, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W,
                       int R, const int32_t* widx, const float* wk, const int32_t* ridx,
                       const float* rw, const float* v, const float* alpha, const float* beta,
                       float* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  ScanArgs A{B * H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta, out, 0};
  // tile = 128 bytes of a row (the whole row when it is shorter)
  const int cols = dtype == 0 ? (d_v < 32 ? d_v : 32) : (d_v < 64 ? d_v : 64);
  A.ntiles = d_v / cols;
  if (dtype == 0) {
    if (d_v == 16) return launch<float, 16>(M, A, stream);
    return launch<float, 32>(M, A, stream);
  }
  if (d_v == 16) return launch<uint16_t, 16>(M, A, stream);
  if (d_v == 32) return launch<uint16_t, 32>(M, A, stream);
  return launch<uint16_t, 64>(M, A, stream);
}

}  // namespace sdm
