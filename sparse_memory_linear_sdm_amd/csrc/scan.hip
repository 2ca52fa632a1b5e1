// Scan kernel: T sequential steps of the gated delta write and the sparse
// read (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)", section
// "Meccanismo Core", items 3 and 4) for every (b,h) memory.
//
// Layout and parallelism.  The update is independent per column, so each
// memory's d_v columns are split into tiles of 32 columns (128 bytes of an
// fp32 row = one cache line; 64 bytes of a bf16 row, which keeps the same
// number of workgroups as fp32 -- measured faster than 128-byte bf16 tiles
// at half the workgroups); one workgroup owns one (b,h,tile) and walks
// t = 0..T-1.  Blocks
// are numbered so that all tiles of one memory land on the same XCD (blocks
// are dealt to the 8 XCDs round-robin), so a memory's index, weight and value
// traffic is fetched into one L2.  Nothing here is a dense contraction, so
// there is no MFMA: the kernel is bound by HBM traffic, (2W + R) tile rows
// per step per tile, all random accesses of one tile row each.
//
// Two wavefronts per workgroup:
//   producer  stages each step's metadata into an LDS "plan", two chunks of
//             kChunk steps ahead of the consumer (triple buffer): the byte
//             offsets of the W write rows and R read rows in the tile, their
//             weights, the tile's v columns, alpha and beta.  It also resolves
//             every read-after-write hazard inside the consumer's prefetch
//             window: for each row of step u, the newest step s in
//             [u - D, u] (s < u for write rows) writing the same row.  Each
//             step's write set is recorded as a bitmap of hashed rows; a row
//             whose bit is clear in every window bitmap has no hazard (one LDS
//             read per row and window step, no per-lane loops).  The rare
//             candidates are resolved exactly with wave-uniform ballots
//             against the window's write rows kept in registers.  The plan
//             then names, per row, where its current value lives, and marks
//             in the writing step which updated rows a later step will need.
//   consumer  keeps the row gathers of D steps in flight in a register ring:
//             at step u it issues the 16-byte buffer loads of step u + D, then
//             updates step u's W rows (Mt = alpha*M; M = Mt + (beta*k)(v - Mt)
//             in fp32, rounded to the state type) and stores them, and
//             accumulates the R read rows.  Rows the plan forwards come from a
//             small LDS ring of saved updated rows instead of the (possibly
//             stale) loaded values.  Loads of step u + D are issued after the
//             stores of every step before u by the same wavefront, so the
//             only rows they can miss are those written in [u, u + D - 1] --
//             exactly the window the producer checks.  The read's cross-lane
//             sum is deferred: per-lane partial sums go to LDS and are reduced
//             for a whole chunk at once with a transposed lane mapping.
// Memory operations on the state are raw buffer instructions whose offsets
// are never branched around: an invalid row gets an offset past the buffer
// range (loads return zero, stores are dropped), which keeps the compiler's
// count of outstanding loads exact, so the prefetch survives.
// The two waves meet at one workgroup barrier per chunk.
#include "device_common.h"
#include "internal.h"

namespace sdm {
namespace {

constexpr int kChunk = 8;     // steps per plan chunk
constexpr int kNBuf = 3;      // plan chunks resident (consumer: c, c+1; producer: c+2)
constexpr int kBmBits = 14;   // bits of a step's write-set bitmap index (2 KiB per step)
constexpr int kBmWords = (1 << kBmBits) / 32;
// Buffer descriptor word 3 for raw (untyped) buffer access on gfx9-family GPUs.
constexpr int kBufWord3 = 0x00020000;
// Byte offset outside every buffer range the kernel builds (one memory slice
// is below 2^31 bytes): loads there return zero and stores are dropped.
constexpr uint32_t kOffNone = 0x80000000u;

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

template <typename DT, int COLS>
struct Tile {
  static constexpr int ES = sizeof(DT);
  static constexpr int TB = COLS * ES;     // tile bytes (<= 128)
  static constexpr int EPL = 16 / ES;      // elements per lane per 16-byte access
  static constexpr int LPR = TB / 16;      // lanes per row
  static constexpr int RPI = kWave / LPR;  // rows per wave instruction
  static constexpr int NI = 64 / RPI;      // instructions for 64 rows
};

// Per-step plan.  Row entries are stored transposed: entry [lr][k] describes
// row slot j = k * RPI + lr, so a consumer lane reads its NI rows
// contiguously.  wsrc / rsrc: 0 = the loaded value is current; otherwise
// src - 1 = ring * 64 + j' names updated row j' of the step in LDS ring slot
// `ring`.  wsave bit j: write slot j's updated row is needed by a later step
// of the window (or by this step's read) and must be kept in the ring.
template <int COLS>
struct StepPlan {
  uint32_t wofs[64];
  uint32_t rofs[64];
  float wk[64];
  float rw[64];
  uint16_t wsrc[64];
  uint16_t rsrc[64];
  uint64_t wsave;
  uint32_t fwd;  // nonzero when some row of this step is forwarded
  float a, b;
  float pad;
  float v[COLS];
};

template <typename DT, int COLS, int D>
struct ScanShared {
  using TL = Tile<DT, COLS>;
  StepPlan<COLS> plan[kNBuf][kChunk];
  uint4 upd[D + 1][64 * TL::LPR];            // saved updated rows, as stored
  float part[kChunk][TL::RPI][COLS];          // per-lane partial read sums
  uint32_t bm[D + 1][kBmWords];               // producer: write-set bitmaps
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

__device__ __forceinline__ uint32_t row_hash(uint32_t row) {
  return (row * 2654435761u) >> (32 - kBmBits);
}

template <typename DT>
__device__ __forceinline__ void unpack(const u32x4v& q, float (&f)[16 / sizeof(DT)]) {
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
__device__ __forceinline__ u32x4v pack(const float (&f)[16 / sizeof(DT)]) {
  if constexpr (sizeof(DT) == 4) {
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
  const uint32_t row_bytes = (uint32_t)(A.d_v * (int)sizeof(DT));
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
    StepPlan<COLS>& p = P[s];
    const bool wvalid = lane < A.W && (uint32_t)wi[s] < Nu;
    const bool rvalid = lane < A.R && (uint32_t)ri[s] < Nu;
    const int32_t wrow = wvalid ? wi[s] : -1;
    const uint32_t hw = row_hash((uint32_t)wi[s]), hr = row_hash((uint32_t)ri[s]);
    // write rows: window steps u-1 .. u-D (read before this step's bitmap
    // slot, which held step u-D-1, is recycled)
    bool wcand = false;
#pragma unroll
    for (int a = 1; a <= D; ++a) {
      const int sl = (int)((u - a + (D + 1)) % (D + 1));
      const uint32_t word = sh.bm[sl][hw >> 5];
      wcand |= (u - a >= 0) && ((word >> (hw & 31)) & 1u);
    }
    wcand = wcand && wvalid;
    uint4* clr = reinterpret_cast<uint4*>(sh.bm[cur]);
    clr[lane] = make_uint4(0, 0, 0, 0);
    clr[lane + kWave] = make_uint4(0, 0, 0, 0);
    if (lane == 0) p.wsave = 0;
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
    // exact resolution of the candidates, newest writer first; the writer
    // step is told to keep that row in the ring
    uint32_t wsrc = 0, rsrc = 0;
    for (uint64_t m = __ballot(wcand); m; m &= m - 1) {
      const int L = __ffsll((unsigned long long)m) - 1;
      const int32_t row = __builtin_amdgcn_readlane(wi[s], L);
#pragma unroll
      for (int a = 1; a <= D; ++a) {
        const uint64_t hit = __ballot(ring.prev[a - 1] == row);
        if (hit) {
          const int jj = __ffsll((unsigned long long)hit) - 1;
          const int64_t sw = u - a;
          const uint32_t src = 1 + (uint32_t)(sw % (D + 1)) * 64 + (uint32_t)jj;
          if (lane == L) wsrc = src;
          if (lane == 0) sh.plan[(sw / kChunk) % kNBuf][sw % kChunk].wsave |= 1ull << jj;
          break;
        }
      }
      wave_sync();
    }
    for (uint64_t m = __ballot(rcand); m; m &= m - 1) {
      const int L = __ffsll((unsigned long long)m) - 1;
      const int32_t row = __builtin_amdgcn_readlane(ri[s], L);
#pragma unroll
      for (int a = 0; a <= D; ++a) {
        const uint64_t hit = __ballot((a == 0 ? wrow : ring.prev[a > 0 ? a - 1 : 0]) == row);
        if (hit) {
          const int jj = __ffsll((unsigned long long)hit) - 1;
          const int64_t sw = u - a;
          const uint32_t src = 1 + (uint32_t)(sw % (D + 1)) * 64 + (uint32_t)jj;
          if (lane == L) rsrc = src;
          if (lane == 0) sh.plan[(sw / kChunk) % kNBuf][sw % kChunk].wsave |= 1ull << jj;
          break;
        }
      }
      wave_sync();
    }
#pragma unroll
    for (int a = D - 1; a > 0; --a) ring.prev[a] = ring.prev[a - 1];
    ring.prev[0] = wrow;
    p.wofs[tslot] = wvalid ? (uint32_t)wi[s] * row_bytes : kOffNone;
    p.rofs[tslot] = rvalid ? (uint32_t)ri[s] * row_bytes : kOffNone;
    p.wk[tslot] = wkv[s];
    p.rw[tslot] = rvalid ? rwv[s] : 0.0f;
    p.wsrc[tslot] = (uint16_t)wsrc;
    p.rsrc[tslot] = (uint16_t)rsrc;
    const bool anyfwd = __ballot(wsrc != 0 || rsrc != 0) != 0;
    if (lane == 0) {
      p.fwd = anyfwd ? 1u : 0u;
      p.a = ab[s];
    }
    if (lane == 1) p.b = ab[s];
    if (lane < COLS) p.v[lane] = vv[s];
  }
}

// ---------------------------------------------------------------- consumer

template <typename DT, int COLS, int D>
struct Consumer {
  using TL = Tile<DT, COLS>;
  static constexpr int NI = TL::NI, EPL = TL::EPL, LPR = TL::LPR, RPI = TL::RPI;

  u32x4v wv[D + 1][NI];
  u32x4v rv[D + 1][NI];
  __amdgpu_buffer_rsrc_t mres;  // this memory's tile column, range = the memory slice
  uint32_t lane_off;             // lc * 16

  __device__ __forceinline__ const StepPlan<COLS>& plan(ScanShared<DT, COLS, D>& sh,
                                                        int64_t u) const {
    return sh.plan[(u / kChunk) % kNBuf][u % kChunk];
  }

  // Gathers of step u (nothing is fetched when u is past the end).
  template <int SLOT>
  __device__ __forceinline__ void issue(ScanShared<DT, COLS, D>& sh, int lr, int64_t u,
                                        int64_t T) {
    const StepPlan<COLS>& p = plan(sh, u);
    const bool live = u < T;
    uint32_t wo[NI], ro[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const uint32_t w = p.wofs[lr * NI + k], r = p.rofs[lr * NI + k];
      wo[k] = live ? w + lane_off : kOffNone;
      ro[k] = live ? r + lane_off : kOffNone;
    }
#pragma unroll
    for (int k = 0; k < NI; ++k)
      wv[SLOT][k] = __builtin_amdgcn_raw_buffer_load_b128(mres, wo[k], 0, 0);
#pragma unroll
    for (int k = 0; k < NI; ++k)
      rv[SLOT][k] = __builtin_amdgcn_raw_buffer_load_b128(mres, ro[k], 0, 0);
  }

  // Sum the chunk's per-lane partials into out: lane g handles float4 group
  // g of the chunk's kChunk x COLS outputs.
  __device__ __forceinline__ void reduce_chunk(ScanShared<DT, COLS, D>& sh, float* out_mem,
                                               int d_v, int64_t T, int tile, int64_t t0) {
    constexpr int G4 = COLS / 4;
    const int lane = lane_id();
#pragma unroll
    for (int g0 = 0; g0 < kChunk * G4; g0 += kWave) {
      const int g = g0 + lane;
      if (g < kChunk * G4) {
        const int s = g / G4, c4 = g % G4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int r = 0; r < RPI; ++r) {
          const float4 x = *reinterpret_cast<const float4*>(&sh.part[s][r][c4 * 4]);
          acc.x += x.x;
          acc.y += x.y;
          acc.z += x.z;
          acc.w += x.w;
        }
        if (t0 + s < T)
          *reinterpret_cast<float4*>(out_mem + (t0 + s) * d_v + tile * COLS + c4 * 4) = acc;
      }
    }
  }

  template <int SLOT>
  __device__ __forceinline__ void step(ScanShared<DT, COLS, D>& sh, float* out_mem, int d_v,
                                       int64_t T, int tile, int lr, int lc, int64_t u) {
    issue<(SLOT + D) % (D + 1)>(sh, lr, u + D, T);
    const StepPlan<COLS>& p = plan(sh, u);
    uint32_t wo[NI];
    float wkk[NI], rwk[NI], vv[EPL];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      wo[k] = p.wofs[lr * NI + k] + lane_off;  // kOffNone + lane_off is still out of range
      wkk[k] = p.wk[lr * NI + k];
      rwk[k] = p.rw[lr * NI + k];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) vv[e] = p.v[lc * EPL + e];
    const float a = p.a, b = p.b;
    const uint32_t fwd = p.fwd;
    const uint64_t save = p.wsave;
    if (fwd) {  // rare: take forwarded rows from the ring
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const uint32_t src = p.wsrc[lr * NI + k];
        if (src) wv[SLOT][k] = lds_u4(sh.upd[(src - 1) >> 6][((src - 1) & 63) * LPR + lc]);
      }
    }
    // gated delta write
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      float m[EPL];
      unpack<DT>(wv[SLOT][k], m);
      const float g = b * wkk[k];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float mt = a * m[e];
        m[e] = fmaf(g, vv[e] - mt, mt);
      }
      wv[SLOT][k] = pack<DT>(m);
      __builtin_amdgcn_raw_buffer_store_b128(wv[SLOT][k], mres, wo[k], 0, 0);
    }
    if (save) {  // rare: keep the rows a later step (or this read) needs
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int j = k * RPI + lr;
        if ((save >> j) & 1ull) {
          const u32x4v q = wv[SLOT][k];
          sh.upd[SLOT][j * LPR + lc] = make_uint4(q.x, q.y, q.z, q.w);
        }
      }
      wave_sync();
    }
    if (fwd) {
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const uint32_t src = p.rsrc[lr * NI + k];
        if (src) rv[SLOT][k] = lds_u4(sh.upd[(src - 1) >> 6][((src - 1) & 63) * LPR + lc]);
      }
    }
    // sparse read (invalid rows carry weight 0 and load as zero)
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      float m[EPL];
      unpack<DT>(rv[SLOT][k], m);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(rwk[k], m[e], acc[e]);
    }
    float* dst = &sh.part[u % kChunk][lr][lc * EPL];
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    // end of a plan chunk (the last one may be partial): reduce its reads,
    // then meet the producer, which passes one barrier per chunk
    if ((u % kChunk) == kChunk - 1 || u == T - 1) {
      wave_sync();
      reduce_chunk(sh, out_mem, d_v, T, tile, u - (u % kChunk));
      __syncthreads();
    }
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
  DT* const Mm = M + (int64_t)mem * A.N * d_v;
  float* const out_mem = A.out + (int64_t)mem * T * d_v;
  Consumer<DT, COLS, D> cs;
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
    cs.template step<0>(sh, out_mem, d_v, T, tile, lr, lc, u);
    cs.template step<1 % (D + 1)>(sh, out_mem, d_v, T, tile, lr, lc, u + 1);
    if constexpr (D >= 2) cs.template step<2 % (D + 1)>(sh, out_mem, d_v, T, tile, lr, lc, u + 2);
    if constexpr (D >= 3) cs.template step<3 % (D + 1)>(sh, out_mem, d_v, T, tile, lr, lc, u + 3);
  }
  // tail: fewer than D + 1 steps
  if (u < T) cs.template step<0>(sh, out_mem, d_v, T, tile, lr, lc, u);
  if (u + 1 < T) cs.template step<1 % (D + 1)>(sh, out_mem, d_v, T, tile, lr, lc, u + 1);
  if constexpr (D >= 3) {
    if (u + 2 < T) cs.template step<2 % (D + 1)>(sh, out_mem, d_v, T, tile, lr, lc, u + 2);
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
  // tile = 32 columns of a row (the whole row when it is shorter)
  const int cols = d_v < 32 ? d_v : 32;
  A.ntiles = d_v / cols;
  if (dtype == 0) {
    if (d_v == 16) return launch<float, 16>(M, A, stream);
    return launch<float, 32>(M, A, stream);
  }
  if (d_v == 16) return launch<uint16_t, 16>(M, A, stream);
  return launch<uint16_t, 32>(M, A, stream);
}

}  // namespace sdm
