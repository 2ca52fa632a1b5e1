// Scan kernel: T sequential steps of the gated delta write and the sparse
// read (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)", section
// "Meccanismo Core", items 3 and 4) for every (b,h) memory.
//
// Layout and parallelism.  The update is independent per column, so each
// memory's d_v columns are split into tiles of 32 columns (128 bytes of an
// fp32 row = one cache line; 64 bytes of a bf16 row and 32 bytes of an fp8
// E4M3 row, which keep the same number of workgroups as fp32 -- measured
// faster than line-sized bf16 or fp8 tiles at a half or a quarter of the
// workgroups); one workgroup owns one (b,h,tile) and walks t = 0..T-1.  With few memories (narrow 16-column tiles and still room on
// the chip) the rows of a memory are further split between two workgroups by
// a hash of the row index; each adds its part of the read into the zeroed
// output.  Blocks are numbered so that all tiles and shards of one memory
// land on the same XCD (blocks are dealt to the 8 XCDs round-robin), so a
// memory's index, weight and value traffic, and the rows its tiles share,
// are fetched into one L2.  Nothing here is a dense contraction, so
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
//             whose bit is clear in every window bitmap has no hazard.  The
//             rare candidates are resolved exactly with wave-uniform ballots
//             against the window's write rows kept in registers.  The plan
//             then names, per row, where its current value lives, and marks
//             in the writing step which updated rows a later step will need.
//             A chunk is handled in batches (clear its bitmaps, set them, probe
//             them, resolve, write the plan), so the producer pays a few LDS
//             round trips per chunk rather than per step, and the metadata of
//             the next chunk is loaded while the current one is processed.
//   consumer  keeps the row gathers of D steps in flight in a register ring:
//             at step u it issues the 16-byte buffer loads of step u + D, then
//             updates step u's W rows (Mt = alpha*M; M = Mt + (beta*k)(v - Mt)
//             in fp32, rounded to the state type; for fp8 in a fixed
//             binary32 order with no contraction) and stores them, and
//             accumulates the R read rows.  The training variant (SAVE)
//             also stores each write row's current value, before the update,
//             and each row the read uses, after it, to the tape the reverse
//             pass reads (so that pass never touches M).  Rows the plan forwards come
//             from a small LDS ring of saved updated rows instead of the
//             (possibly stale) loaded values.  Loads of step u + D are issued after the
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
#include "ranges.h"
#include "scan_rows.h"

namespace sdm {
namespace {

constexpr int kChunk = 8;     // steps per plan chunk
constexpr int kNBuf = 3;      // plan chunks resident (consumer: c, c+1; producer: c+2)
constexpr int kBmBits = 14;   // bits of a step's write-set bitmap index (2 KiB per step)
constexpr int kBmWords = (1 << kBmBits) / 32;
constexpr int kBmSlots = 2 * kChunk;  // bitmaps of the last two chunks' steps, slot = u % 16
// Buffer descriptor word 3 for raw (untyped) buffer access on gfx9-family GPUs.
constexpr int kBufWord3 = 0x00020000;
// Byte offset outside every buffer range the kernel builds (ranges.h: every
// range is below 2^31 bytes): loads there return zero and stores are dropped.
constexpr uint32_t kOffNone = ranges::kOffNone;

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
// contiguously.  src: low half for the write row, high half for the read
// row; 0 = the loaded value is current, otherwise src - 1 = ring * 64 + j'
// names updated row j' of the step in LDS ring slot `ring`.  wsave bit j:
// write slot j's updated row is needed by a later step of the window (or by
// this step's read) and must be kept in the ring.  Every producer lane writes
// one entry of v and sc (entries past COLS, and sc past 2, are unused), so
// the plan is written without branches.
enum { kScAlpha = 0, kScBeta = 1, kScFwd = 2 };
template <int COLS>
struct StepPlan {
  uint32_t wofs[64];
  uint32_t rofs[64];
  float wk[64];
  float rw[64];
  uint32_t src[64];
  float v[64];
  uint32_t sc[64];  // alpha, beta (float bits), forward flag
  uint64_t wsave;
  uint64_t pad;
};

template <typename DT, int COLS, int D>
struct ScanShared {
  using TL = Tile<DT, COLS>;
  StepPlan<COLS> plan[kNBuf][kChunk];
  uint4 upd[D + 1][64 * TL::LPR];            // saved updated rows, as stored
  float part[kChunk][TL::RPI][COLS];          // per-lane partial read sums
  uint32_t bm[kBmSlots][kBmWords];            // producer: write-set bitmaps
  int32_t wrows[kBmSlots][64];                // producer: write rows, slot = u % 16
  int32_t rrows[kChunk][64];                  // producer: read rows of the current chunk
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
  void* tape;  // training forward: [n_mem, T, W + R, d_v] in the state type: per step the
              // W pre-write rows, then the R rows the read used
  int ntiles;
  int shards;  // 1, or 2: rows split between two workgroups by row_shard()
};

// Row sharding (few memories): the workgroups of one (memory, tile) pair
// split the rows by a hash of the row index, so each row is always handled by
// the same workgroup and all hazard reasoning stays inside one workgroup.
__device__ __forceinline__ uint32_t row_shard(uint32_t row) { return (row * 0xC2B2AE35u) >> 31; }

// Write-set filter: a row sets three bits of one 32-bit word of the step's
// bitmap (word and bit positions from two multiplicative hashes), and a probe
// is a candidate only when all three are set.  Set and probe are one LDS
// operation each; with ~64 rows per 512-word bitmap a probe of an absent row
// is a false candidate about once in 10^4 (two bits: once in 10^3).
struct RowKey {
  uint32_t word, mask;
};
__device__ __forceinline__ RowKey row_key(uint32_t row) {
  const uint32_t h1 = row * 2654435761u, h2 = row * 0x85EBCA77u;
  return RowKey{h1 >> (32 - (kBmBits - 5)),
                (1u << (h2 >> 27)) | (1u << ((h2 >> 22) & 31u)) | (1u << ((h2 >> 17) & 31u))};
}

// ---------------------------------------------------------------- producer

// One chunk's metadata as loaded by the producer wave: lane j holds write
// slot j and read slot j of every step; lanes < COLS hold v; lanes 0, 1 hold
// alpha, beta.
struct ChunkMeta {
  int32_t wi[kChunk], ri[kChunk];
  float wk[kChunk], rw[kChunk], v[kChunk], ab[kChunk];
};

template <typename DT, int COLS, int D>
struct Producer {
  using TL = Tile<DT, COLS>;

  // Issue the loads of chunk c; no wait here.  Branch-free: every address is
  // clamped into its array (steps past the end read the chunk's last step,
  // lanes past W, R or COLS read lane 0), and produce() masks those entries by
  // step and lane.  A chunk wholly past the end loads nothing.
  __device__ __forceinline__ void load(ChunkMeta& m, const ScanArgs& A, int mem, int tile,
                                       int64_t c) const {
    const int64_t t0 = c * kChunk;
    if (t0 >= A.T) return;  // never read: produce() returns before using m
    const int lane = lane_id();
    const int last = (int)((A.T - t0) < kChunk ? (A.T - t0) : kChunk) - 1;
    const int64_t base = (int64_t)mem * A.T + t0;
    const int32_t* const pwi = A.widx + base * A.W + (lane < A.W ? lane : 0);
    const float* const pwk = A.wk + base * A.W + (lane < A.W ? lane : 0);
    const int32_t* const pri = A.ridx + base * A.R + (lane < A.R ? lane : 0);
    const float* const prw = A.rw + base * A.R + (lane < A.R ? lane : 0);
    const float* const pv = A.v + base * A.d_v + (int64_t)tile * COLS + (lane < COLS ? lane : 0);
    const float* const pab = (lane == 1 ? A.beta : A.alpha) + base;
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const int ss = s < last ? s : last;
      m.wi[s] = pwi[ss * A.W];
      m.wk[s] = pwk[ss * A.W];
      m.ri[s] = pri[ss * A.R];
      m.rw[s] = prw[ss * A.R];
      m.v[s] = pv[(int64_t)ss * A.d_v];
      m.ab[s] = pab[ss];
    }
  }

  // Build the plan of chunk c from its loaded metadata.
  int shard;  // this workgroup's row shard (0 when the rows are not split)

  __device__ __forceinline__ bool owns(int32_t row, int shards) const {
    return shards == 1 || row_shard((uint32_t)row) == (uint32_t)shard;
  }

  __device__ __forceinline__ void produce(ScanShared<DT, COLS, D>& sh, const ChunkMeta& m,
                                          const ScanArgs& A, int64_t c) {
    const int lane = lane_id();
    const int64_t t0 = c * kChunk;
    if (t0 >= A.T) return;
    const int steps = (int)((A.T - t0) < kChunk ? (A.T - t0) : kChunk);
    StepPlan<COLS>* P = sh.plan[c % kNBuf];
    const uint32_t Nu = (uint32_t)A.N;
    const uint32_t row_bytes = (uint32_t)(A.d_v * (int)sizeof(DT));
    const int slot0 = (int)(t0 % kBmSlots);  // 0 or kChunk
    int32_t wrow[kChunk], rrow[kChunk];
    RowKey hw[kChunk], hr[kChunk];
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      // rows of another shard are handled like empty slots
      const bool wv = s < steps && lane < A.W && (uint32_t)m.wi[s] < Nu && owns(m.wi[s], A.shards);
      const bool rv = s < steps && lane < A.R && (uint32_t)m.ri[s] < Nu && owns(m.ri[s], A.shards);
      wrow[s] = wv ? m.wi[s] : -1;
      rrow[s] = rv ? m.ri[s] : -1;
      hw[s] = row_key((uint32_t)m.wi[s]);
      hr[s] = row_key((uint32_t)m.ri[s]);
    }
    // 1. clear this chunk's bitmaps (they held the steps of chunk c - 2) and
    //    the wsave masks of its steps
    {
      uint4* clr = reinterpret_cast<uint4*>(sh.bm[slot0]);
      constexpr int kVec = kChunk * kBmWords / 4;
#pragma unroll
      for (int i = 0; i < kVec / kWave; ++i) clr[i * kWave + lane] = make_uint4(0, 0, 0, 0);
      P[lane & (kChunk - 1)].wsave = 0;  // every lane clears one mask; all 8 get cleared
    }
    wave_sync();
    // 2. record each step's write set, and stage its rows for exact checks
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      atomicOr(&sh.bm[slot0 + s][hw[s].word], wrow[s] >= 0 ? hw[s].mask : 0u);
      sh.wrows[slot0 + s][lane] = wrow[s];
      sh.rrows[s][lane] = rrow[s];
    }
    wave_sync();
    // 3. probe: write rows against steps u-1 .. u-D, read rows against u .. u-D
    uint32_t wcand = 0, rcand = 0;  // bit s: this lane's row of step s is a candidate
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const int64_t u = t0 + s;
      bool wc = false, rc = false;
#pragma unroll
      for (int a = 0; a <= D; ++a) {
        const int sl = (slot0 + s - a + kBmSlots) % kBmSlots;
        const bool live = u - a >= 0;
        if (a > 0) wc |= live && (sh.bm[sl][hw[s].word] & hw[s].mask) == hw[s].mask;
        rc |= live && (sh.bm[sl][hr[s].word] & hr[s].mask) == hr[s].mask;
      }
      wcand |= (wc && wrow[s] >= 0) ? (1u << s) : 0u;
      rcand |= (rc && rrow[s] >= 0) ? (1u << s) : 0u;
    }
    // 4. the plan, with every row taken as loaded
    const int lr = lane % TL::RPI, k = lane / TL::RPI;
    const int tslot = lr * TL::NI + k;  // transposed position of row slot j = lane
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      if (s < steps) {
        StepPlan<COLS>& p = P[s];
        p.wofs[tslot] = wrow[s] >= 0 ? (uint32_t)wrow[s] * row_bytes : kOffNone;
        p.rofs[tslot] = rrow[s] >= 0 ? (uint32_t)rrow[s] * row_bytes : kOffNone;
        p.wk[tslot] = m.wk[s];
        p.rw[tslot] = rrow[s] >= 0 ? m.rw[s] : 0.0f;
        p.v[lane] = m.v[s];  // src is read only when the step is flagged, and then written by resolve()
        p.sc[lane] = lane == kScFwd ? 0u : __float_as_uint(m.ab[s]);
      }
    }
    wave_sync();
    // 5. exact resolution of the (rare) candidates, newest writer first: the
    //    row's source in the plan becomes the writer's ring entry, the step
    //    is flagged, and the writer step is told to keep that row
    if (__ballot((wcand | rcand) != 0u) != 0ull) resolve(sh, wcand, rcand, t0, steps, slot0, tslot);
  }

  // Steps with candidates only.  For such a step the write rows of its
  // window (steps u - D .. u) are read from LDS once, all together; each
  // candidate then takes the newest matching writer with one ballot per
  // window step.  Every lane writes its src entry of a flagged step.
  __device__ void resolve(ScanShared<DT, COLS, D>& sh, uint32_t wcand, uint32_t rcand,
                          int64_t t0, int steps, int slot0, int tslot) {
    const int lane = lane_id();
    uint32_t todo = 0;  // bit s: step s has a candidate
#pragma unroll
    for (int s = 0; s < kChunk; ++s)
      todo |= __ballot(((wcand | rcand) >> s) & 1u) != 0ull ? 1u << s : 0u;
#pragma unroll 1
    for (; todo; todo &= todo - 1) {
      const int s = __ffs(todo) - 1;
      if (s >= steps) break;
      const int64_t u = t0 + s;
      int32_t win[D + 1];  // write rows of steps u - a, one per lane
#pragma unroll
      for (int a = 0; a <= D; ++a) win[a] = sh.wrows[(slot0 + s - a + kBmSlots) % kBmSlots][lane];
      const uint64_t wm = __ballot((wcand >> s) & 1u), rm = __ballot((rcand >> s) & 1u);
      uint32_t src = 0;
      for (int pass = 0; pass < 2; ++pass) {  // write rows (a >= 1), then read rows (a >= 0)
        for (uint64_t mk = pass == 0 ? wm : rm; mk; mk &= mk - 1) {
          const int L = __ffsll((unsigned long long)mk) - 1;
          const int32_t row = pass == 0 ? sh.wrows[slot0 + s][L] : sh.rrows[s][L];
#pragma unroll
          for (int a = 0; a <= D; ++a) {
            if (a < 1 - pass || u - a < 0) continue;
            const uint64_t hit = __ballot(win[a] == row);
            if (hit) {
              const int jj = __ffsll((unsigned long long)hit) - 1;
              const int64_t sw = u - a;
              const uint32_t code = 1 + (uint32_t)(sw % (D + 1)) * 64 + (uint32_t)jj;
              if (lane == L) src |= pass == 0 ? code : code << 16;
              if (lane == 0) sh.plan[(sw / kChunk) % kNBuf][sw % kChunk].wsave |= 1ull << jj;
              break;
            }
          }
        }
      }
      if (__ballot(src != 0u) != 0ull) {
        StepPlan<COLS>& p = sh.plan[(u / kChunk) % kNBuf][u % kChunk];
        p.src[tslot] = src;
        if (lane == 0) p.sc[kScFwd] = 1u;
      }
    }
    wave_sync();
  }
};

// ---------------------------------------------------------------- consumer

template <typename DT, int COLS, int D, bool SAVE>
struct Consumer {
  using TL = Tile<DT, COLS>;
  static constexpr int NI = TL::NI, EPL = TL::EPL, LPR = TL::LPR, RPI = TL::RPI;

  u32x4v wv[D + 1][NI];
  u32x4v rv[D + 1][NI];
  __amdgpu_buffer_rsrc_t mres;  // this memory's tile column, range = the memory slice
  __amdgpu_buffer_rsrc_t tres;  // SAVE: this memory's tape slice, shifted to the tile column
  uint32_t tape_step;            // SAVE: bytes of one step's W + R tape rows
  uint32_t read_base;            // SAVE: bytes before a step's first read row (W rows)
  uint32_t row_bytes;            // SAVE: bytes of one full row
  uint32_t lane_off;             // lc * 16
  bool accumulate;               // rows split over two workgroups: add into out

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
  // With two row shards each adds its partial sum to the zeroed output; two
  // additions onto zero give the same bits in either order.
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
        if (t0 + s < T) {
          float* const o = out_mem + (t0 + s) * d_v + tile * COLS + c4 * 4;
          if (accumulate) {
            unsafeAtomicAdd(o + 0, acc.x);
            unsafeAtomicAdd(o + 1, acc.y);
            unsafeAtomicAdd(o + 2, acc.z);
            unsafeAtomicAdd(o + 3, acc.w);
          } else {
            *reinterpret_cast<float4*>(o) = acc;
          }
        }
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
    const float a = __uint_as_float(p.sc[kScAlpha]), b = __uint_as_float(p.sc[kScBeta]);
    const uint32_t fwd = p.sc[kScFwd];
    const uint64_t save = p.wsave;
    if (fwd) {  // rare: take forwarded rows from the ring
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const uint32_t src = p.src[lr * NI + k] & 0xFFFFu;
        if (src) wv[SLOT][k] = lds_u4(sh.upd[(src - 1) >> 6][((src - 1) & 63) * LPR + lc]);
      }
    }
    if constexpr (SAVE) {  // the pre-write rows, as stored, for the reverse pass
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const uint32_t to = p.wofs[lr * NI + k] == kOffNone
                                ? kOffNone
                                : (uint32_t)u * tape_step + (uint32_t)(k * RPI + lr) * row_bytes +
                                      lane_off;
        __builtin_amdgcn_raw_buffer_store_b128(wv[SLOT][k], tres, to, 0, 0);
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
        if constexpr (sizeof(DT) == 1) {
          m[e] = write_elem_exact(a, g, vv[e], m[e]);
        } else {
          const float mt = a * m[e];
          m[e] = fmaf(g, vv[e] - mt, mt);
        }
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
        const uint32_t src = p.src[lr * NI + k] >> 16;
        if (src) rv[SLOT][k] = lds_u4(sh.upd[(src - 1) >> 6][((src - 1) & 63) * LPR + lc]);
      }
    }
    if constexpr (SAVE) {  // the rows the read uses, for the reverse pass
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const uint32_t to = p.rofs[lr * NI + k] == kOffNone
                                ? kOffNone
                                : (uint32_t)u * tape_step + read_base +
                                      (uint32_t)(k * RPI + lr) * row_bytes + lane_off;
        __builtin_amdgcn_raw_buffer_store_b128(rv[SLOT][k], tres, to, 0, 0);
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

  // Gathers of steps 0 .. D-1.  Each is followed by NI stores to an offset
  // past the buffer range (dropped by the hardware), so that the memory
  // operations enter the loop in the same pattern as a step leaves them (a
  // step's gathers, then its stores).  The compiler's wait counts at the loop
  // head are the tighter of the two paths into it; without this they would be
  // sized for the store-free prologue and wait on the next step's gathers.
  template <int S>
  __device__ __forceinline__ void prologue(ScanShared<DT, COLS, D>& sh, int lr, int64_t T) {
    if constexpr (S < D) {
      issue<S>(sh, lr, S, T);
      const u32x4v zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < (SAVE ? 3 : 1) * NI; ++k)  // distinct offsets: identical stores would be merged
        __builtin_amdgcn_raw_buffer_store_b128(zero, mres, kOffNone + (uint32_t)(S * 3 * NI + k) * 16u,
                                               0, 0);
      prologue<S + 1>(sh, lr, T);
    }
  }

  // Steps u .. u + D (u a multiple of D + 1, so step u + S uses ring slot S).
  template <int S>
  __device__ __forceinline__ void round(ScanShared<DT, COLS, D>& sh, float* out_mem, int d_v,
                                        int64_t T, int tile, int lr, int lc, int64_t u) {
    if constexpr (S <= D) {
      step<S>(sh, out_mem, d_v, T, tile, lr, lc, u + S);
      round<S + 1>(sh, out_mem, d_v, T, tile, lr, lc, u);
    }
  }

  // The last steps (fewer than D + 1) from u on.
  template <int S>
  __device__ __forceinline__ void tail(ScanShared<DT, COLS, D>& sh, float* out_mem, int d_v,
                                       int64_t T, int tile, int lr, int lc, int64_t u) {
    if constexpr (S < D) {
      if (u + S < T) {
        step<S>(sh, out_mem, d_v, T, tile, lr, lc, u + S);
        tail<S + 1>(sh, out_mem, d_v, T, tile, lr, lc, u);
      }
    }
  }
};

template <typename DT, int COLS, int D, bool SAVE>
__global__ __launch_bounds__(2 * kWave) void scan_kernel(DT* __restrict__ M, ScanArgs A) {
  using TL = Tile<DT, COLS>;
  __shared__ ScanShared<DT, COLS, D> sh;

  // XCD-aware numbering: bid = (((g * shards) + shard) * ntiles + tile) * 8 + x,
  // memory = g*8 + x, so every tile and shard of a memory shares one XCD's L2.
  const int bid = blockIdx.x;
  const int x = bid & 7;
  const int rest = bid >> 3;
  const int tile = rest % A.ntiles;
  const int shard = (rest / A.ntiles) % A.shards;
  const int mem = (rest / A.ntiles / A.shards) * 8 + x;
  if (mem >= A.n_mem) return;  // whole workgroup leaves together

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t T = A.T;
  const int64_t nchunks = (T + kChunk - 1) / kChunk;

  if (wave == 1) {
    // producer: chunks 0 and 1 before the consumer starts, then chunk c + 2
    // while the consumer runs chunk c; the metadata of the next chunk is in
    // flight while one is processed (two register sets, loop unrolled by 2)
    Producer<DT, COLS, D> pr;
    pr.shard = shard;
    ChunkMeta ma, mb;
    pr.load(ma, A, mem, tile, 0);
    pr.load(mb, A, mem, tile, 1);
    pr.produce(sh, ma, A, 0);
    pr.load(ma, A, mem, tile, 2);
    pr.produce(sh, mb, A, 1);
    __syncthreads();
    for (int64_t c = 0; c < nchunks; c += 2) {
      pr.load(mb, A, mem, tile, c + 3);
      pr.produce(sh, ma, A, c + 2);
      __syncthreads();
      if (c + 1 < nchunks) {
        pr.load(ma, A, mem, tile, c + 4);
        pr.produce(sh, mb, A, c + 3);
        __syncthreads();
      }
    }
    return;
  }

  // consumer
  const int lr = lane / TL::LPR;
  const int lc = lane % TL::LPR;
  const int d_v = A.d_v;
  DT* const Mm = M + (int64_t)mem * A.N * d_v;
  float* const out_mem = A.out + (int64_t)mem * T * d_v;
  Consumer<DT, COLS, D, SAVE> cs;
  cs.lane_off = (uint32_t)(lc * 16);
  cs.accumulate = A.shards > 1;
  // descriptor ranges from ranges.h (checked on the host before the launch)
  const int64_t row_bytes = (int64_t)d_v * (int64_t)sizeof(DT);
  if constexpr (SAVE) {
    const int64_t tape_rows = T * (A.W + A.R);  // rows of one memory's tape
    cs.tape_step = (uint32_t)((A.W + A.R) * row_bytes);
    cs.read_base = (uint32_t)(A.W * row_bytes);
    cs.row_bytes = (uint32_t)row_bytes;
    cs.tres = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<DT*>(A.tape) + (int64_t)mem * tape_rows * d_v + (int64_t)tile * COLS, 0,
        (int)ranges::table_range(tape_rows, row_bytes, tile, TL::TB), kBufWord3);
  }
  cs.mres = __builtin_amdgcn_make_buffer_rsrc(
      Mm + (int64_t)tile * COLS, 0, (int)ranges::table_range(A.N, row_bytes, tile, TL::TB),
      kBufWord3);
  __syncthreads();
  cs.template prologue<0>(sh, lr, T);
  int64_t u = 0;
  for (; u + D + 1 <= T; u += D + 1) cs.template round<0>(sh, out_mem, d_v, T, tile, lr, lc, u);
  cs.template tail<0>(sh, out_mem, d_v, T, tile, lr, lc, u);
}

__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ p, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename DT, int COLS, int D, bool SAVE>
hipError_t launch(void* M, ScanArgs A, hipStream_t stream) {
  static_assert(D >= 1 && D <= kChunk, "prefetch depth");
  static_assert((SAVE ? 5 : 3) * Tile<DT, COLS>::NI * D <= 63,
                "outstanding vector memory operations");
  A.ntiles = A.d_v / COLS;
  if (!ranges::scan_tiles_ok(A.N, A.d_v, (int)sizeof(DT), A.T, A.W, A.R, COLS, SAVE))
    return hipErrorInvalidValue;  // never taken: the C-ABI layer checked every tile width
  const int groups = (A.n_mem + 7) / 8;
  const int64_t blocks = (int64_t)groups * A.shards * A.ntiles * 8;
  if (A.shards > 1) {  // the shards add into out
    const int64_t n4 = (int64_t)A.n_mem * A.T * A.d_v / 4;
    const int64_t zb = (n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)zb), dim3(256), 0, stream,
                       reinterpret_cast<float4*>(A.out), n4);
  }
  hipLaunchKernelGGL((scan_kernel<DT, COLS, D, SAVE>), dim3((unsigned)blocks), dim3(2 * kWave), 0,
                     stream, reinterpret_cast<DT*>(M), A);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

}  // namespace

hipError_t launch_scan(void* M, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W,
                       int R, const int32_t* widx, const float* wk, const int32_t* ridx,
                       const float* rw, const float* v, const float* alpha, const float* beta,
                       float* out, void* tape, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  ScanArgs A{B * H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta, out, tape, 0, 1};
  // Tile width and prefetch depth, measured on the mid (64 memories) and
  // long-stream (16 memories) workloads.  Each workgroup walks its steps at a
  // rate set by the latency of a step's gathers, so with few memories the
  // chip is filled by splitting rows into more, narrower tiles (16 columns),
  // whose fewer memory instructions per step leave room for a deeper
  // prefetch.  When 16-column tiles would need more workgroups than there
  // are compute units, 32-column tiles with one step in flight are fastest.
  // With room for twice as many narrow workgroups still, each (memory, tile)
  // is split into two row shards on two compute units: a step's gathers are
  // then spread over twice the units, and the tiles of one memory, which
  // fetch the same rows at about the same time, share them in L2 (long-stream
  // scan 2.27 -> 2.82 TB/s; three steps in flight are then best for fp32 too).
  const int cus = compute_units();
  const bool narrow = d_v == 16 || (int64_t)A.n_mem * (d_v / 16) <= cus;
  if (dtype != 2 && narrow && 2 * (int64_t)A.n_mem * (d_v / 16) <= cus) A.shards = 2;
  if (tape) {  // training forward (fp32 state): also keep the pre-write and the read rows
    if (!narrow) return launch<float, 32, 1, true>(M, A, stream);
    if (A.shards == 2) return launch<float, 16, 3, true>(M, A, stream);
    return launch<float, 16, 2, true>(M, A, stream);
  }
  if (dtype == 0) {
    if (!narrow) return launch<float, 32, 1, false>(M, A, stream);
    if (A.shards == 2) return launch<float, 16, 3, false>(M, A, stream);
    return launch<float, 16, 2, false>(M, A, stream);
  }
  if (dtype == 2) {  // fp8 E4M3: 32-column tiles (32-byte rows)
    const bool few = (int64_t)A.n_mem * (d_v / 32) < cus;
    if (!few) return launch<fp8e4m3, 32, 1, false>(M, A, stream);
    if (2 * (int64_t)A.n_mem * (d_v / 32) <= cus) A.shards = 2;
    return launch<fp8e4m3, 32, 3, false>(M, A, stream);
  }
  if (!narrow) return launch<uint16_t, 32, 1, false>(M, A, stream);
  return launch<uint16_t, 16, 3, false>(M, A, stream);
}

}  // namespace sdm
