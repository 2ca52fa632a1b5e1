// Planned scan: the T steps of sdm_scan (page "Riepilogo Tecnico: Sparse
// Delta Memory (SDM)", section "Meccanismo Core", items 3 and 4) for fp32
// state, with the per-step planning taken out of the scan workgroups.
//
// Why.  With few memories (the long-stream workload: 16 memories of 2^20
// rows) the scan can only fill the chip by splitting each memory's rows
// between several workgroups ("row shards").  Each step's W + R rows are
// random, so a shard owns a fraction of them; if every (tile, shard)
// workgroup plans its own step (offsets, its shard's rows, read-after-write
// hazards) it examines all W + R rows, and its gathers are as many
// mostly-empty instructions as an unsharded step needs.  Here a separate
// pass plans each step once per memory and writes, per shard, compacted
// lists; the scan workgroups only read their shard's lists, so their
// gathers cover whole 128-byte rows (32 fp32 columns: one cache line) with
// a fraction of the instructions.
//
//   plan     (plan_kernel) one 256-thread workgroup per (memory, 32 steps).
//            Per step: each row's shard (a multiplicative hash of the row
//            index), its position in its shard's compacted list (ballots),
//            and the list entries (row, weight).  Read-after-write hazards:
//            every write row of the workgroup's steps and of the
//            kPlanLookback steps before them goes into an LDS hash table
//            (row -> step, position) and sets a bit of an LDS filter; a
//            row of step u looks up the newest step in [u - kPlanLookback,
//            u] (write rows: [.., u - 1]) that writes it (the filter
//            answers the rows no window step writes, nearly all of them,
//            with one read), and the entry's source names that step's
//            offset a and list position.  Flagged (memory, shard, step)
//            entries get their source lists written; the rest do not.
//   scan     (planned_kernel) one workgroup per (memory, 32-column tile,
//            shard), two wavefronts, at most two workgroups per CU.  A
//            loader wavefront copies each chunk (8 or 16 steps) of the
//            shard's lists into an LDS plan (byte offsets and weights laid
//            out per row group, sources, v columns, gates) two chunks
//            ahead, with the loads of the next chunk in flight.  The
//            consumer wavefront runs a chunk per loop iteration with every
//            step index known at compile time, keeps the gathers of D steps
//            in flight with NIC instructions per list (8 rows each), and
//            reads each step's plan one step ahead.  Every updated row goes
//            into an LDS ring of the last D + 1 steps, and a flagged step
//            takes the rows its sources name from the ring instead of the
//            (stale) gathered values.  A step whose list is longer than the
//            fast path's NIC * 8 rows, or whose source lies past the ring,
//            takes a synchronous path (wait for every access, then gather,
//            write, wait, read).  Row traffic is raw buffer instructions
//            with out-of-range offsets for empty slots, as in the scan
//            kernel, and non-temporal.
//   combine  (combine_kernel) with S > 1 shards each shard's read sums go to
//            its own partial output, and out = p_0 + p_1 + ... + p_{S-1},
//            added in that fixed order, so results do not depend on timing.
#include "device_common.h"
#include "internal.h"
#include "planned.h"
#include "ranges.h"
#include "scan_rows.h"

namespace sdm {
namespace {

constexpr int kCols = 32;             // fp32 columns per tile: one 128-byte line of a row
constexpr int kCpolNT = 2;            // buffer instruction cache policy: nt (non-temporal)
constexpr int kTileBytes = kCols * 4;
constexpr int kLPR = kTileBytes / 16;  // lanes per row (8)
constexpr int kRPI = kWave / kLPR;     // rows per wave instruction (8)
constexpr int kNI = 64 / kRPI;         // instructions for 64 rows (8)
constexpr int kNBuf = 3;               // plan chunks resident
constexpr int kBufWord3 = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kOffNone = ranges::kOffNone;

constexpr int kWin = kPlanSteps + kPlanLookback;  // steps a plan workgroup looks at
constexpr int kHashBits = 12;
constexpr int kHashCap = 1 << kHashBits;  // > kWin * 64 / 0.6: probes stay short
constexpr uint32_t kEmpty = 0xFFFFFFFFu;  // rows are < 2^31

enum : uint32_t { kFlagFwd = 1u };

__device__ __forceinline__ uint32_t shard_of(uint32_t row, int sbits) {
  return sbits ? (row * 0xC2B2AE35u) >> (32 - sbits) : 0u;
}

__device__ __forceinline__ uint32_t hash_slot(uint32_t row) {
  return (row * 2654435761u) >> (32 - kHashBits);
}

// ------------------------------------------------------------------- plan

struct PlanArgs {
  int n_mem, S, sbits, W, R;
  int64_t N, T, nblk;
  const int32_t* widx;
  const float* wk;
  const int32_t* ridx;
  const float* rw;
  uint32_t* hdr;
  uint2* went;
  uint2* rent;
  uint16_t* srcw;
  uint16_t* srcr;
};

constexpr int kFiltBits = 15;  // bit filter over the window's write rows (4 KiB)

struct PlanShared {
  uint32_t hrow[kHashCap];  // hash table of the window's write rows: row (kEmpty: free) ...
  uint16_t hinf[kHashCap];  // ... and window step << 8 | list position
  uint32_t filt[(1 << kFiltBits) / 32];  // bit filt_bit(row) set for every row in the table
};
static_assert(kWin <= 255, "window steps fit the high byte of a 16-bit hinf entry");

__device__ __forceinline__ uint32_t filt_bit(uint32_t row) {
  return (row * 0x85EBCA77u) >> (32 - kFiltBits);
}

// Source code of the newest write of `row` in window steps [lo, hi], or 0.
// Almost every row has none: the filter answers those with one read.
__device__ __forceinline__ uint32_t newest_writer(const PlanShared& sh, uint32_t row, int lo,
                                                  int hi, int ls) {
  const uint32_t f = filt_bit(row);
  if (((sh.filt[f >> 5] >> (f & 31u)) & 1u) == 0u) return 0u;
  int best = -1;
  uint32_t pos = 0;
  for (uint32_t p = hash_slot(row);; p = (p + 1) & (kHashCap - 1)) {
    const uint32_t r = sh.hrow[p];
    if (r == kEmpty) break;
    if (r == row) {
      const uint32_t inf = sh.hinf[p];
      const int s = (int)(inf >> 8);
      if (s >= lo && s <= hi && s > best) {
        best = s;
        pos = inf & 0xFFu;
      }
    }
  }
  return best < 0 ? 0u : 1u + (uint32_t)(ls - best) * 64u + pos;
}

// Lane j's position among the valid lanes of its shard (lanes below j), and
// for lane s < S the number of valid lanes in shard s: the lanes of a shard
// are those that agree on each of the sbits shard bits.
__device__ __forceinline__ void shard_positions(bool valid, uint32_t shard, int sbits, int lane,
                                                int* pos, int* count) {
  const uint64_t below = (1ull << lane) - 1ull;
  const uint64_t vm = __ballot(valid);
  uint64_t mine = vm, lanes_s = vm;
  for (int b = 0; b < sbits; ++b) {
    const uint64_t m = __ballot(valid && ((shard >> b) & 1u));
    mine &= ((shard >> b) & 1u) ? m : ~m;
    lanes_s &= (((uint32_t)lane >> b) & 1u) ? m : ~m;
  }
  *pos = __popcll(mine & below);
  *count = __popcll(lanes_s);
}

__global__ __launch_bounds__(256) void plan_kernel(PlanArgs A) {
  __shared__ PlanShared sh;
  const int64_t bid = blockIdx.x;
  const int mem = (int)(bid / A.nblk);
  const int64_t t0 = (bid % A.nblk) * kPlanSteps;
  const int own = (int)(A.T - t0 < kPlanSteps ? A.T - t0 : kPlanSteps);
  const int lb = (int)(t0 < kPlanLookback ? t0 : kPlanLookback);
  const int nwin = lb + own;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const uint32_t Nu = (uint32_t)A.N;  // N < 2^31
  const int64_t T = A.T;

  for (int i = tid; i < kHashCap; i += 256) sh.hrow[i] = kEmpty;
  for (int i = tid; i < (1 << kFiltBits) / 32; i += 256) sh.filt[i] = 0u;
  __syncthreads();

  // 1. every window step: rows, shards, list positions, hash inserts; for the
  //    workgroup's own steps also the list entries and the counts.  A wave
  //    takes window steps w, w + 4, ... (in both phases: the lookback is 0
  //    or 8 steps, so a step's wave is the same in phase 2 and what phase 2
  //    needs stays in registers); all of its loads are issued first, so it
  //    waits for memory once rather than once per step.
  constexpr int kPer = (kWin + 3) / 4;
  int32_t wrow_r[kPer], rrow_r[kPer];
  float wk_r[kPer], rw_r[kPer];
  uint8_t wpos_r[kPer], rpos_r[kPer];
  uint32_t cnt_r[kPer];  // lane s < S: write count | read count << 8 of shard s
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ls = w + 4 * i;
    const int64_t st = (int64_t)mem * T + (t0 - lb + ls);
    const bool live = ls < nwin, own_step = live && ls >= lb;
    wrow_r[i] = (live && lane < A.W) ? A.widx[st * A.W + lane] : -1;
    wk_r[i] = (live && lane < A.W) ? A.wk[st * A.W + lane] : 0.0f;
    rrow_r[i] = (own_step && lane < A.R) ? A.ridx[st * A.R + lane] : -1;
    rw_r[i] = (own_step && lane < A.R) ? A.rw[st * A.R + lane] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ls = w + 4 * i;
    if (ls >= nwin) break;
    const int64_t ts = t0 - lb + ls;
    const int32_t row = wrow_r[i];
    const bool ok = (uint32_t)row < Nu;
    const uint32_t sh_w = shard_of((uint32_t)row, A.sbits);
    int pos, cw;
    shard_positions(ok, sh_w, A.sbits, lane, &pos, &cw);
    wrow_r[i] = ok ? row : -1;
    wpos_r[i] = (uint8_t)pos;
    if (ok) {
      const uint32_t inf = ((uint32_t)ls << 8) | (uint32_t)pos;
      for (uint32_t p = hash_slot((uint32_t)row);; p = (p + 1) & (kHashCap - 1)) {
        if (atomicCAS(&sh.hrow[p], kEmpty, (uint32_t)row) == kEmpty) {
          sh.hinf[p] = (uint16_t)inf;
          break;
        }
      }
      const uint32_t f = filt_bit((uint32_t)row);
      atomicOr(&sh.filt[f >> 5], 1u << (f & 31u));
    }
    cnt_r[i] = 0u;
    if (ls >= lb) {
      if (ok) {
        const int64_t e = (((int64_t)mem * A.S + sh_w) * T + ts) * 64 + pos;
        A.went[e] = make_uint2((uint32_t)row, __float_as_uint(wk_r[i]));
      }
      const int32_t rr = rrow_r[i];
      const bool rok = (uint32_t)rr < Nu;
      const uint32_t sh_r = shard_of((uint32_t)rr, A.sbits);
      int rp, cr;
      shard_positions(rok, sh_r, A.sbits, lane, &rp, &cr);
      rrow_r[i] = rok ? rr : -1;
      rpos_r[i] = (uint8_t)rp;
      if (rok) {
        const int64_t e = (((int64_t)mem * A.S + sh_r) * T + ts) * 64 + rp;
        A.rent[e] = make_uint2((uint32_t)rr, __float_as_uint(rw_r[i]));
      }
      cnt_r[i] = (uint32_t)cw | ((uint32_t)cr << 8);
    }
  }
  __syncthreads();

  // 2. sources of every own step's rows, the flags and the headers
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ls = w + 4 * i;
    if (ls >= nwin) break;
    if (ls < lb) continue;
    const int64_t ts = t0 - lb + ls;
    const int32_t row = wrow_r[i];
    const int32_t rr = rrow_r[i];
    const uint32_t sw = row >= 0 ? newest_writer(sh, (uint32_t)row, ls - kPlanLookback, ls - 1, ls) : 0u;
    const uint32_t sr = rr >= 0 ? newest_writer(sh, (uint32_t)rr, ls - kPlanLookback, ls, ls) : 0u;
    uint32_t fwd = 0;  // lane s < S: shard s has a forwarded row in this step
    if (__ballot(sw != 0u || sr != 0u) != 0ull) {  // rare: some row has a writer in the window
      const uint32_t sh_w = shard_of((uint32_t)row, A.sbits), sh_r = shard_of((uint32_t)rr, A.sbits);
      for (int s = 0; s < A.S; ++s) {
        const bool mine_w = row >= 0 && sh_w == (uint32_t)s;
        const bool mine_r = rr >= 0 && sh_r == (uint32_t)s;
        const bool f = __ballot((mine_w && sw != 0u) || (mine_r && sr != 0u)) != 0ull;
        if (lane == s) fwd = f ? 1u : 0u;
        if (f) {
          const int64_t base = (((int64_t)mem * A.S + s) * T + ts) * 64;
          if (mine_w) A.srcw[base + wpos_r[i]] = (uint16_t)sw;
          if (mine_r) A.srcr[base + rpos_r[i]] = (uint16_t)sr;
        }
      }
    }
    if (lane < A.S) A.hdr[((int64_t)mem * A.S + lane) * T + ts] = cnt_r[i] | (fwd << 16);
  }
}

// ------------------------------------------------------------------- scan

// One step of a shard's plan in LDS: the first C = NIC * kRPI positions of
// its write and read lists (the fast path's capacity), laid out for the
// consumer lanes that use them.  List position k * kRPI + lr belongs to the
// lanes of row group lr; rec[lr] holds, for k < NIC, the write offsets, the
// read offsets, the write weights and the read weights (bit patterns), so a
// lane reads its whole step with NIC 16-byte LDS reads.  src[lr][k]: write
// source (low half) | read source << 16, valid when the step is flagged.
template <int NIC>
struct PStep {
  uint32_t rec[kRPI][4 * NIC];
  uint32_t src[kRPI][NIC];
  float v[kCols];
  float alpha, beta;
  uint32_t flags;  // kFlagFwd | kFlagSync | write count << 8 | read count << 16
  uint32_t pad;
};

template <int D, int NIC, int kChunk>
struct PShared {
  static constexpr int C = NIC * kRPI;
  PStep<NIC> plan[kNBuf][kChunk];
  uint4 upd[D + 1][C * kLPR];       // updated rows of the last D + 1 steps, by list position
  float part[kChunk][kRPI][kCols];  // per-lane partial read sums
};

struct PScanArgs {
  int n_mem, S, ntiles, d_v;
  int64_t N, T;
  const uint32_t* hdr;
  const uint2* went;
  const uint2* rent;
  const uint16_t* srcw;
  const uint16_t* srcr;
  const float* v;
  const float* alpha;
  const float* beta;
  float* out;  // S == 1: [n_mem, T, d_v]; otherwise the partials [S, n_mem, T, d_v]
};

// A step goes through the synchronous path when a list is longer than C or
// when a row's newest writer inside the prefetch window put it at a list
// position >= C (so it is not in the ring).
enum : uint32_t { kFlagSync = 4u };

// One chunk's plan data as the loader wavefront loads it: lane s < kChunk
// holds step s's header; every lane j < C holds list position j of each
// step (loaded whatever the list length, so no load waits for a header;
// positions past the length are masked when the plan is written).
template <int kChunk>
struct ChunkRegs {
  uint32_t h, al, be;  // lane s < kChunk: step s's header, alpha, beta
  u32x2 we[kChunk], re[kChunk];
  uint32_t sw[kChunk], sr[kChunk];
  uint32_t vv[kChunk];
};

// Loader wavefront: the loads of chunk q + 1 are in flight while chunk q is
// written into the LDS plan (two register sets).  Every load is a raw
// buffer load through a descriptor over this workgroup's slice of an array,
// so a masked lane is an out-of-range offset rather than a branch.
template <int D, int NIC, int kChunk>
struct Loader {
  static constexpr int C = NIC * kRPI;
  __amdgpu_buffer_rsrc_t rhdr, rwent, rrent, rsrcw, rsrcr, rv, ralpha, rbeta;
  uint32_t off_list, off_src, off_v;  // this lane's byte offset within a step (or kOffNone)
  uint32_t step_v;                            // bytes between steps of v

  __device__ __forceinline__ void init(const PScanArgs& A, int mem, int tile, int64_t ubase) {
    const int lane = lane_id();
    const int64_t T = A.T;
    rhdr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(A.hdr + ubase), 0, (int)(T * 4), kBufWord3);
    rwent = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint2*>(A.went + ubase * 64), 0, (int)(T * 512), kBufWord3);
    rrent = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint2*>(A.rent + ubase * 64), 0, (int)(T * 512), kBufWord3);
    rsrcw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A.srcw + ubase * 64), 0, (int)(T * 128), kBufWord3);
    rsrcr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A.srcr + ubase * 64), 0, (int)(T * 128), kBufWord3);
    rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(A.v + (int64_t)mem * T * A.d_v + (int64_t)tile * kCols), 0,
                                           (int)(T * A.d_v * 4 - (int64_t)tile * kCols * 4), kBufWord3);
    ralpha = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(A.alpha + (int64_t)mem * T), 0, (int)(T * 4), kBufWord3);
    rbeta = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(A.beta + (int64_t)mem * T), 0, (int)(T * 4), kBufWord3);
    off_list = lane < C ? (uint32_t)lane * 8u : kOffNone;
    off_src = lane < C ? (uint32_t)lane * 2u : kOffNone;
    off_v = lane < kCols ? (uint32_t)lane * 4u : kOffNone;
    step_v = (uint32_t)A.d_v * 4u;
  }

  // Issue the loads of chunk q; no wait.  Steps past the end load nothing
  // (their offsets are out of range).
  __device__ __forceinline__ void load(ChunkRegs<kChunk>& r, const PScanArgs& A, int64_t q) const {
    const int64_t t0 = q * kChunk;
    const int lane = lane_id();
    const uint32_t th = (lane < kChunk && t0 + lane < A.T) ? (uint32_t)(t0 + lane) * 4u : kOffNone;
    r.h = __builtin_amdgcn_raw_buffer_load_b32(rhdr, th, 0, 0);
    r.al = __builtin_amdgcn_raw_buffer_load_b32(ralpha, th, 0, 0);
    r.be = __builtin_amdgcn_raw_buffer_load_b32(rbeta, th, 0, 0);
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      const bool live = t0 + s < A.T;
      const uint32_t t = (uint32_t)(t0 + s);
      const uint32_t ol = live ? off_list + t * 512u : kOffNone;  // kOffNone + x stays out of range
      const uint32_t os = live ? off_src + t * 128u : kOffNone;
      r.we[s] = __builtin_amdgcn_raw_buffer_load_b64(rwent, ol, 0, 0);
      r.re[s] = __builtin_amdgcn_raw_buffer_load_b64(rrent, ol, 0, 0);
      r.sw[s] = __builtin_amdgcn_raw_buffer_load_b16(rsrcw, os, 0, 0);
      r.sr[s] = __builtin_amdgcn_raw_buffer_load_b16(rsrcr, os, 0, 0);
      r.vv[s] = __builtin_amdgcn_raw_buffer_load_b32(rv, live ? off_v + t * step_v : kOffNone, 0, 0);
    }
  }

  // true when a source names a writer inside the window at a position the
  // ring does not hold
  __device__ static __forceinline__ bool beyond_ring(uint32_t code, int amin) {
    const int at = (int)((code - 1u) >> 6);
    return code != 0u && at >= amin && at <= D && ((code - 1u) & 63u) >= (uint32_t)C;
  }

  // Write chunk q's plan from its loaded data.  Entries past a list's length
  // and the sources of unflagged steps (never written by the plan pass) are
  // masked here.
  __device__ __forceinline__ void fill(PShared<D, NIC, kChunk>& sh, const PScanArgs& A, const ChunkRegs<kChunk>& r,
                                       int64_t q) const {
    const int64_t t0 = q * kChunk;
    if (t0 >= A.T) return;
    const int steps = (int)(A.T - t0 < kChunk ? A.T - t0 : kChunk);
    const int lane = lane_id();
    const uint32_t Nu = (uint32_t)A.N;
    const uint32_t row_bytes = (uint32_t)A.d_v * 4u;
    const int lr = lane % kRPI, k = lane / kRPI;  // for lanes < C: list position k * kRPI + lr
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
      if (s < steps) {
        PStep<NIC>& p = sh.plan[q % kNBuf][s];
        const uint32_t hs = (uint32_t)__builtin_amdgcn_readlane((int)r.h, s);
        const int nw = (int)(hs & 0xFFu), nr = (int)((hs >> 8) & 0xFFu);
        const bool fwd = ((hs >> 16) & 1u) != 0u;
        const uint32_t wrow = r.we[s].x, rrow = r.re[s].x;
        const bool wok = lane < nw && wrow < Nu;  // rows at or past N: skipped
        const bool rok = lane < nr && rrow < Nu;
        if (lane < C) {
          p.rec[lr][k] = wok ? wrow * row_bytes : kOffNone;
          p.rec[lr][NIC + k] = rok ? rrow * row_bytes : kOffNone;
          p.rec[lr][2 * NIC + k] = r.we[s].y;
          p.rec[lr][3 * NIC + k] = rok ? r.re[s].y : 0u;
        }
        if (lane < kCols) p.v[lane] = __uint_as_float(r.vv[s]);
        bool far = false;
        if (fwd) {  // rare: the sources of a flagged step
          const uint32_t sw = lane < nw ? (r.sw[s] & 0xFFFFu) : 0u;
          const uint32_t sr = lane < nr ? (r.sr[s] & 0xFFFFu) : 0u;
          if (lane < C) p.src[lr][k] = sw | (sr << 16);
          far = __ballot(lane < C && (beyond_ring(sw, 1) || beyond_ring(sr, 0))) != 0ull;
        }
        const uint32_t al = (uint32_t)__builtin_amdgcn_readlane((int)r.al, s);
        const uint32_t be = (uint32_t)__builtin_amdgcn_readlane((int)r.be, s);
        if (lane == 0) {
          p.alpha = __uint_as_float(al);
          p.beta = __uint_as_float(be);
          p.flags = (fwd ? kFlagFwd : 0u) | ((nw > C || nr > C || far) ? kFlagSync : 0u) |
                    ((uint32_t)nw << 8) | ((uint32_t)nr << 16);
        }
      }
    }
  }
};

// Consumer wavefront.  The loop body is one plan chunk of kChunk steps with
// the step index known at compile time (D + 1 divides kChunk, so a step's
// ring slot is too); the gathers of step s + D are issued at step s.
template <int D, int NIC, int kChunk>
struct PConsumer {
  static constexpr int C = NIC * kRPI;
  static_assert(kChunk % (D + 1) == 0, "ring slots repeat within a chunk");
  static_assert(NIC % 2 == 0, "offsets of a step are NIC / 2 16-byte reads");
  u32x4v wv[D + 1][NIC];
  u32x4v rv[D + 1][NIC];
  // Plan words read one step ahead, kept exactly as loaded: whatever is
  // computed from them happens where they are used, a step later, so no
  // step waits for the LDS read it just issued.
  uint32_t gw[NIC], gr[NIC];  // row offsets of the next gathers
  bool glive;                 // those gathers' step is inside the sequence
  uint32_t cw[NIC];           // the next step's write offsets ...
  uint32_t ck[NIC], cr[NIC];  // ... weights (bit patterns) ...
  float4 cv;                  // ... v columns ...
  float ca, cb;               // ... gates ...
  uint32_t cf;                // ... and flags
  __amdgpu_buffer_rsrc_t mres;  // this memory's tile column, range = the memory's table
  uint32_t lane_off;            // lc * 16
  int lr, lc;
  // the synchronous path reads the shard's lists from the workspace
  const uint2* went;
  const uint2* rent;
  int64_t ubase;
  uint32_t Nu, row_bytes;

  // ring slot of the step `a` steps before a step in slot `slot`
  __device__ static __forceinline__ int ring(int slot, int a) { return (slot - a + D + 1) % (D + 1); }

  __device__ __forceinline__ void read_gather_offsets(const PStep<NIC>& p, bool live) {
    const uint4* r = reinterpret_cast<const uint4*>(p.rec[lr]);
#pragma unroll
    for (int i = 0; i < NIC / 2; ++i) {
      const uint4 x = r[i];
      const uint32_t o[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * i + e;
        if (j < NIC) gw[j] = o[e];
        else gr[j - NIC] = o[e];
      }
    }
    glive = live;
  }

  __device__ __forceinline__ void read_step_fields(const PStep<NIC>& p) {
    const uint4* r = reinterpret_cast<const uint4*>(p.rec[lr]);
#pragma unroll
    for (int i = 0; i < NIC; ++i) {
      const uint4 x = r[i];
      const uint32_t o[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * i + e;
        if (j < NIC) cw[j] = o[e];
        else if (j >= 2 * NIC && j < 3 * NIC) ck[j - 2 * NIC] = o[e];
        else if (j >= 3 * NIC) cr[j - 3 * NIC] = o[e];
      }
    }
    cv = *reinterpret_cast<const float4*>(&p.v[lc * 4]);
    ca = p.alpha;
    cb = p.beta;
    cf = p.flags;
  }

  template <int SLOT>
  __device__ __forceinline__ void issue() {
    uint32_t ow[NIC], orr[NIC];
#pragma unroll
    for (int k = 0; k < NIC; ++k) {  // kOffNone + lane_off is still out of range
      ow[k] = glive ? gw[k] + lane_off : kOffNone;
      orr[k] = glive ? gr[k] + lane_off : kOffNone;
    }
    // Row pieces are used once per step and rarely again while a cache
    // would hold them: the gathers and the stores of the rows are
    // non-temporal (cache policy nt), which leaves L2 to the plan lists and
    // v that the workgroups of a memory share.
#pragma unroll
    for (int k = 0; k < NIC; ++k)
      wv[SLOT][k] = __builtin_amdgcn_raw_buffer_load_b128(mres, ow[k], 0, kCpolNT);
#pragma unroll
    for (int k = 0; k < NIC; ++k)
      rv[SLOT][k] = __builtin_amdgcn_raw_buffer_load_b128(mres, orr[k], 0, kCpolNT);
  }

  // A whole step without the prefetch (rare): wait for every earlier
  // access, gather the write rows (all list positions, entries read from the
  // workspace), update and store them, wait, then gather and sum the read
  // rows, so every value is current.  Rows at positions < C also go into the
  // ring for the later steps whose gathers are already in flight.
  template <int SLOT>
  __device__ __forceinline__ void sync_step(PShared<D, NIC, kChunk>& sh, int64_t u, uint32_t nw,
                                            uint32_t nr, float a, float b, const float (&vv)[4],
                                            float (&acc)[4]) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    const int64_t e0 = (ubase + u) * 64;
    uint32_t off[kNI];
    float wt[kNI];
    u32x4v q[kNI];
#pragma unroll
    for (int k = 0; k < kNI; ++k) {
      const uint32_t j = (uint32_t)(k * kRPI + lr);
      const uint2 en = j < nw ? went[e0 + j] : make_uint2(kEmpty, 0u);
      off[k] = (en.x < Nu ? en.x * row_bytes : kOffNone) + lane_off;
      wt[k] = __uint_as_float(en.y);
    }
#pragma unroll
    for (int k = 0; k < kNI; ++k) q[k] = __builtin_amdgcn_raw_buffer_load_b128(mres, off[k], 0, 0);
#pragma unroll
    for (int k = 0; k < kNI; ++k) {
      float m[4];
      unpack<float>(q[k], m);
      const float g = b * wt[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = write_elem<float>(a, g, vv[e], m[e]);
      q[k] = pack<float>(m);
      __builtin_amdgcn_raw_buffer_store_b128(q[k], mres, off[k], 0, 0);
      if (k < NIC) sh.upd[SLOT][(k * kRPI + lr) * kLPR + lc] = make_uint4(q[k].x, q[k].y, q[k].z, q[k].w);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the stores are done before the read's gathers
#pragma unroll
    for (int k = 0; k < kNI; ++k) {
      const uint32_t j = (uint32_t)(k * kRPI + lr);
      const uint2 en = j < nr ? rent[e0 + j] : make_uint2(kEmpty, 0u);
      off[k] = (en.x < Nu ? en.x * row_bytes : kOffNone) + lane_off;
      wt[k] = en.x < Nu ? __uint_as_float(en.y) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kNI; ++k) q[k] = __builtin_amdgcn_raw_buffer_load_b128(mres, off[k], 0, 0);
#pragma unroll
    for (int k = 0; k < kNI; ++k) {
      float m[4];
      unpack<float>(q[k], m);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(wt[k], m[e], acc[e]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }

  // Sum a chunk's per-lane partials: lane g handles float4 groups g,
  // g + 64, ... of the chunk's kChunk x kCols outputs.
  __device__ __forceinline__ void reduce_chunk(PShared<D, NIC, kChunk>& sh, float* out_mem, int d_v,
                                               int64_t T, int tile, int64_t t0) {
    constexpr int G4 = kCols / 4;
    static_assert((kChunk * G4) % kWave == 0, "whole float4 groups per lane");
#pragma unroll
    for (int q = 0; q < kChunk * G4 / kWave; ++q) {
      const int g = lane_id() + q * kWave;
      const int s = g / G4, c4 = g % G4;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int r = 0; r < kRPI; ++r) {
        const float4 x = *reinterpret_cast<const float4*>(&sh.part[s][r][c4 * 4]);
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
      }
      if (t0 + s < T) {  // read once, by the combine or the caller: streamed past the caches
        const f32x4 v = {acc.x, acc.y, acc.z, acc.w};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out_mem + (t0 + s) * d_v + tile * kCols + c4 * 4));
      }
    }
  }

  // Step s of the chunk starting at t0 (P: its plan, P1: the next chunk's).
  // FULL: this chunk and the next are wholly inside the sequence, so no
  // step or prefetch needs a bounds check.
  template <int s, bool FULL>
  __device__ __forceinline__ void step(PShared<D, NIC, kChunk>& sh, const PStep<NIC>* P,
                                       const PStep<NIC>* P1, int64_t t0, int64_t T) {
    constexpr int SLOT = s % (D + 1);
    const int64_t u = t0 + s;
    issue<(SLOT + D) % (D + 1)>();
    // offsets of the gathers after these (step s + D + 1), then this step's
    // fields (read during the previous step) and the next step's
    {
      constexpr int g = s + D + 1;
      read_gather_offsets(g < kChunk ? P[g] : P1[g - kChunk], FULL || t0 + g < T);
    }
    uint32_t wo[NIC];
    float wkk[NIC], rwk[NIC];
#pragma unroll
    for (int k = 0; k < NIC; ++k) {
      wo[k] = cw[k] + lane_off;  // kOffNone + lane_off is still out of range
      wkk[k] = __uint_as_float(ck[k]);
      rwk[k] = __uint_as_float(cr[k]);
    }
    const float vv[4] = {cv.x, cv.y, cv.z, cv.w};
    const float a = ca, b = cb;
    const uint32_t flags = __builtin_amdgcn_readfirstlane(cf);
    if (FULL || u + 1 < T) read_step_fields(s + 1 < kChunk ? P[s + 1] : P1[0]);
    const PStep<NIC>& p = P[s];
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (flags & kFlagSync) {
      sync_step<SLOT>(sh, u, (flags >> 8) & 0xFFu, (flags >> 16) & 0xFFu, a, b, vv, acc);
    } else {
      // Rows written inside the prefetch window (rare) come from the ring.
      // They go to registers of their own and are chosen at the point of
      // use: writing a gather register while its load is in flight would
      // make the compiler wait for that load there, and the common path
      // after the branch would inherit the wait.
      const bool fwd = (flags & kFlagFwd) != 0u;
      u32x4v fw[NIC], fr[NIC];
      bool tw[NIC], tr[NIC];
#pragma unroll
      for (int k = 0; k < NIC; ++k) {
        fw[k] = u32x4v{0u, 0u, 0u, 0u};
        fr[k] = fw[k];
        tw[k] = false;
        tr[k] = false;
      }
      if (fwd) {
        wave_sync();  // the ring rows of earlier steps
#pragma unroll
        for (int k = 0; k < NIC; ++k) {
          const uint32_t code = p.src[lr][k] & 0xFFFFu;
          const int at = (int)((code - 1u) >> 6);
          const uint32_t pos = (code - 1u) & 63u;  // < C: the loader flags others for the slow path
          tw[k] = code != 0u && at >= 1 && at <= D && pos < (uint32_t)C;
          fw[k] = lds_u4(sh.upd[ring(SLOT, tw[k] ? at : 1)][(tw[k] ? pos : 0u) * kLPR + lc]);
        }
      }
      // gated delta write; every updated row also goes into the ring
#pragma unroll
      for (int k = 0; k < NIC; ++k) {
        float m[4];
        unpack<float>(tw[k] ? fw[k] : wv[SLOT][k], m);
        const float g = b * wkk[k];
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = write_elem<float>(a, g, vv[e], m[e]);
        wv[SLOT][k] = pack<float>(m);
        __builtin_amdgcn_raw_buffer_store_b128(wv[SLOT][k], mres, wo[k], 0, kCpolNT);
        const u32x4v q = wv[SLOT][k];
        sh.upd[SLOT][(k * kRPI + lr) * kLPR + lc] = make_uint4(q.x, q.y, q.z, q.w);
      }
      if (fwd) {
        wave_sync();  // this step's ring rows
#pragma unroll
        for (int k = 0; k < NIC; ++k) {
          const uint32_t code = p.src[lr][k] >> 16;
          const int at = (int)((code - 1u) >> 6);
          const uint32_t pos = (code - 1u) & 63u;
          tr[k] = code != 0u && at <= D && pos < (uint32_t)C;
          fr[k] = lds_u4(sh.upd[ring(SLOT, tr[k] ? at : 0)][(tr[k] ? pos : 0u) * kLPR + lc]);
        }
      }
      // sparse read (empty slots carry weight 0 and load as zero)
#pragma unroll
      for (int k = 0; k < NIC; ++k) {
        float m[4];
        unpack<float>(tr[k] ? fr[k] : rv[SLOT][k], m);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(rwk[k], m[e], acc[e]);
      }
    }
    *reinterpret_cast<float4*>(&sh.part[s][lr][lc * 4]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }

  // A full chunk of kChunk steps, then its outputs and the barrier the
  // loader meets (one per chunk).
  template <int s, bool FULL>
  __device__ __forceinline__ void steps(PShared<D, NIC, kChunk>& sh, const PStep<NIC>* P,
                                        const PStep<NIC>* P1, int64_t t0, int64_t T) {
    if constexpr (s < kChunk) {
      step<s, FULL>(sh, P, P1, t0, T);
      steps<s + 1, FULL>(sh, P, P1, t0, T);
    }
  }

  // The last, partial chunk: the same steps, each only while t0 + s < T.
  template <int s>
  __device__ __forceinline__ void tail_steps(PShared<D, NIC, kChunk>& sh, const PStep<NIC>* P,
                                             const PStep<NIC>* P1, int64_t t0, int64_t T) {
    if constexpr (s < kChunk) {
      if (t0 + s < T) {
        step<s, false>(sh, P, P1, t0, T);
        tail_steps<s + 1>(sh, P, P1, t0, T);
      }
    }
  }

  __device__ __forceinline__ void end_chunk(PShared<D, NIC, kChunk>& sh, float* out_mem, int d_v,
                                            int64_t T, int tile, int64_t t0) {
    wave_sync();
    reduce_chunk(sh, out_mem, d_v, T, tile, t0);
    __syncthreads();
  }

  // Gathers of steps 0 .. D-1, each followed by NIC stores past the buffer
  // range (dropped), so the memory operations enter the loop in the pattern
  // a step leaves them in (its gathers, then its stores).
  template <int S>
  __device__ __forceinline__ void prologue(PShared<D, NIC, kChunk>& sh, int64_t T) {
    if constexpr (S == 0) read_step_fields(sh.plan[0][0]);
    if constexpr (S < D) {
      read_gather_offsets(sh.plan[0][S], S < T);
      issue<S>();
      const u32x4v zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < NIC; ++k)  // distinct offsets: identical stores would be merged
        __builtin_amdgcn_raw_buffer_store_b128(zero, mres, kOffNone + (uint32_t)(S * NIC + k) * 16u,
                                               0, 0);
      prologue<S + 1>(sh, T);
    }
    if constexpr (S == D) read_gather_offsets(sh.plan[0][D], D < T);
  }
};

template <int D, int NIC, int kChunk>
__global__ __launch_bounds__(2 * kWave) void planned_kernel(float* __restrict__ M, PScanArgs A) {
  __shared__ PShared<D, NIC, kChunk> sh;
  // XCD-aware numbering as in the scan kernel: every tile and shard of a
  // memory on one XCD, so the rows its tiles share come from one L2.
  const int bid = blockIdx.x;
  const int x = bid & 7;
  const int rest = bid >> 3;
  const int tile = rest % A.ntiles;
  const int shard = (rest / A.ntiles) % A.S;
  const int mem = (rest / A.ntiles / A.S) * 8 + x;
  if (mem >= A.n_mem) return;  // whole workgroup leaves together
  // Each workgroup is one long chain of dependent steps, so its waves take
  // the highest issue priority: kernels running beside it (the next
  // chunk's selections) then fill the cycles the chain leaves idle instead
  // of stretching it.
  __builtin_amdgcn_s_setprio(3);

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t T = A.T;
  const int64_t nchunks = (T + kChunk - 1) / kChunk;
  const int64_t ubase = ((int64_t)mem * A.S + shard) * T;

  if (wave == 1) {
    // loader: chunks 0 and 1 before the consumer starts, then chunk c + 2
    // while the consumer runs chunk c (one barrier per chunk, as the
    // consumer); the loads of chunk c + 3 are in flight meanwhile
    Loader<D, NIC, kChunk> ld;
    ld.init(A, mem, tile, ubase);
    ChunkRegs<kChunk> ra, rb;
    ld.load(ra, A, 0);
    ld.load(rb, A, 1);
    ld.fill(sh, A, ra, 0);
    ld.load(ra, A, 2);
    ld.fill(sh, A, rb, 1);
    __syncthreads();
    for (int64_t c = 0; c < nchunks; c += 2) {
      ld.load(rb, A, c + 3);
      ld.fill(sh, A, ra, c + 2);
      __syncthreads();
      if (c + 1 < nchunks) {
        ld.load(ra, A, c + 4);
        ld.fill(sh, A, rb, c + 3);
        __syncthreads();
      }
    }
    return;
  }

  const int d_v = A.d_v;
  float* const out_mem =
      A.out + ((A.S == 1 ? 0 : (int64_t)shard * A.n_mem) + mem) * T * d_v;
  PConsumer<D, NIC, kChunk> cs;
  cs.lr = lane / kLPR;
  cs.lc = lane % kLPR;
  cs.lane_off = (uint32_t)(cs.lc * 16);
  cs.went = A.went;
  cs.rent = A.rent;
  cs.ubase = ubase;
  cs.Nu = (uint32_t)A.N;
  cs.row_bytes = (uint32_t)d_v * 4u;
  const int64_t row_bytes = (int64_t)d_v * 4;
  cs.mres = __builtin_amdgcn_make_buffer_rsrc(
      M + (int64_t)mem * A.N * d_v + (int64_t)tile * kCols, 0,
      (int)ranges::table_range(A.N, row_bytes, tile, kTileBytes), kBufWord3);
  __syncthreads();
  cs.template prologue<0>(sh, T);
  // chunks whose successor is wholly inside the sequence, then the last
  // whole chunk (its successor may be partial), then the partial one
  const int64_t full = T / kChunk;
  int buf = 0;  // plan buffer of chunk c (c % kNBuf)
  int64_t c = 0;
  for (; c + 1 < full; ++c) {
    const int nxt = buf == kNBuf - 1 ? 0 : buf + 1;
    cs.template steps<0, true>(sh, sh.plan[buf], sh.plan[nxt], c * kChunk, T);
    cs.end_chunk(sh, out_mem, d_v, T, tile, c * kChunk);
    buf = nxt;
  }
  if (c < full) {
    const int nxt = buf == kNBuf - 1 ? 0 : buf + 1;
    cs.template steps<0, false>(sh, sh.plan[buf], sh.plan[nxt], c * kChunk, T);
    cs.end_chunk(sh, out_mem, d_v, T, tile, c * kChunk);
    buf = nxt;
    ++c;
  }
  if (c < nchunks) {
    const int nxt = buf == kNBuf - 1 ? 0 : buf + 1;
    cs.template tail_steps<0>(sh, sh.plan[buf], sh.plan[nxt], c * kChunk, T);
    cs.end_chunk(sh, out_mem, d_v, T, tile, c * kChunk);
  }
}

// out = p_0 + p_1 + ... + p_{S-1}, element by element, added in that order.
// Each partial is read once and out written once: non-temporal accesses
// (streamed past the caches), all S loads of a group in flight together.
template <int S>
__global__ __launch_bounds__(256) void combine_kernel(const f32x4* __restrict__ part,
                                                      f32x4* __restrict__ out, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    f32x4 x[S];
#pragma unroll
    for (int s = 0; s < S; ++s) x[s] = __builtin_nontemporal_load(&part[(int64_t)s * n4 + i]);
    f32x4 o = x[0];
#pragma unroll
    for (int s = 1; s < S; ++s) o += x[s];  // p_0 + p_1 + ... in that order
    __builtin_nontemporal_store(o, &out[i]);
  }
}

// A device attribute of the current device, read once per device.
int device_attr(hipDeviceAttribute_t attr, int fallback, int (&cached)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) v = fallback;
    cached[dev] = v;
  }
  return cached[dev];
}

int cu_count() {
  static int cached[64] = {0};
  return device_attr(hipDeviceAttributeMultiprocessorCount, 256, cached);
}

int lds_per_cu() {
  static int cached[64] = {0};
  return device_attr(hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, 160 * 1024, cached);
}

template <int D, int NIC, int kChunk>
hipError_t launch_planned(float* M, const PScanArgs& A, hipStream_t stream) {
  // the offsets of step u + D + 1 are read during step u: at most one
  // chunk ahead of the one the consumer is in (the loader fills two ahead)
  static_assert(D >= 1 && D <= kChunk - 1, "prefetch depth");
  static_assert(kChunk % (D + 1) == 0, "ring slots repeat within a chunk");
  static_assert(D <= kPlanLookback, "the plan names writers up to kPlanLookback steps back");
  static_assert(NIC >= 1 && NIC <= kNI, "instructions per list");
  static_assert(3 * NIC * D <= 63, "outstanding vector memory operations");
  const int groups = (A.n_mem + 7) / 8;
  const int64_t blocks = (int64_t)groups * A.S * A.ntiles * 8;
  // Each workgroup is one chain of dependent steps over the whole call, so
  // the call lasts as long as its slowest chain. When the grid fits two
  // workgroups per CU, each asks for just over a third of the CU's LDS: no
  // CU can then take a third of them, whatever else is dispatched at the
  // same time (kernels beside, such as the next chunk's selections and
  // plan, use the LDS left over).
  size_t dyn = 0;
  if (blocks <= 2 * (int64_t)cu_count()) {
    const size_t third = ((size_t)lds_per_cu() / 3 / 256 + 1) * 256;
    if (third > sizeof(PShared<D, NIC, kChunk>) && third <= 64 * 1024) dyn = third - sizeof(PShared<D, NIC, kChunk>);
  }
  hipLaunchKernelGGL((planned_kernel<D, NIC, kChunk>), dim3((unsigned)blocks), dim3(2 * kWave), dyn, stream,
                     M, A);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; 256 if the
// query fails).
}  // namespace

int planned_shards(int n_mem, int d_v) {
  // One workgroup per (memory, tile) when those fill the compute units; two
  // shards while that still fits one workgroup per unit; else eight, two
  // workgroups per unit (measured on the long-stream shape: four shards at
  // one workgroup per unit were 1.4 times slower, sixteen no faster).
  const int64_t units = (int64_t)n_mem * (d_v / kCols);
  const int64_t cus = cu_count();
  if (units * 2 > cus) return 1;
  if (units * 4 > cus) return 2;
  return 8;
}

hipError_t launch_scan_plan(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                            const int32_t* widx, const float* wk, const int32_t* ridx,
                            const float* rw, void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int n_mem = B * H;
  const int S = planned_shards(n_mem, d_v);
  const PlanLayout L = plan_layout(n_mem, S, T, d_v);
  char* const base = reinterpret_cast<char*>(ws);
  PlanArgs A{};
  A.n_mem = n_mem;
  A.S = S;
  A.sbits = __builtin_ctz((unsigned)S);
  A.W = W;
  A.R = R;
  A.N = N;
  A.T = T;
  A.nblk = (T + kPlanSteps - 1) / kPlanSteps;
  A.widx = widx;
  A.wk = wk;
  A.ridx = ridx;
  A.rw = rw;
  A.hdr = reinterpret_cast<uint32_t*>(base + L.hdr);
  A.went = reinterpret_cast<uint2*>(base + L.went);
  A.rent = reinterpret_cast<uint2*>(base + L.rent);
  A.srcw = reinterpret_cast<uint16_t*>(base + L.srcw);
  A.srcr = reinterpret_cast<uint16_t*>(base + L.srcr);
  const int64_t blocks = (int64_t)n_mem * A.nblk;
  hipLaunchKernelGGL(plan_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, A);
  return hipGetLastError();
}

hipError_t launch_scan_planned(float* M, int B, int H, int64_t N, int d_v, int64_t T,
                               const float* v, const float* alpha, const float* beta, float* out,
                               void* ws, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int n_mem = B * H;
  const int S = planned_shards(n_mem, d_v);
  const PlanLayout L = plan_layout(n_mem, S, T, d_v);
  char* const base = reinterpret_cast<char*>(ws);
  PScanArgs A{};
  A.n_mem = n_mem;
  A.S = S;
  A.ntiles = d_v / kCols;
  A.d_v = d_v;
  A.N = N;
  A.T = T;
  A.hdr = reinterpret_cast<const uint32_t*>(base + L.hdr);
  A.went = reinterpret_cast<const uint2*>(base + L.went);
  A.rent = reinterpret_cast<const uint2*>(base + L.rent);
  A.srcw = reinterpret_cast<const uint16_t*>(base + L.srcw);
  A.srcr = reinterpret_cast<const uint16_t*>(base + L.srcr);
  A.v = v;
  A.alpha = alpha;
  A.beta = beta;
  A.out = S == 1 ? out : reinterpret_cast<float*>(base + L.part);
  if (!ranges::scan_tiles_ok(N, d_v, 4, T, 1, 1, kCols, false))
    return hipErrorInvalidValue;  // never taken: the C-ABI layer checked the tile ranges
  // Fast-path capacity per list (NIC * 8 rows) and prefetch depth per shard
  // count: a shard's share of 64 random rows exceeds 48 (of 2 shards) about
  // once in 10^5 lists and 16 (of 8) about twice in 10^3; longer lists take
  // the synchronous path.  Chunk length: 16 steps where the LDS allows two
  // workgroups per CU with it (one barrier and one output pass per 16
  // steps), else 8.
  hipError_t e;
  if (S == 1) e = launch_planned<1, 8, 8>(M, A, stream);
  else if (S == 2) e = launch_planned<3, 6, 8>(M, A, stream);
  else e = launch_planned<7, 2, 16>(M, A, stream);  // 8 shards
  if (e != hipSuccess || S == 1) return e;
  const int64_t n4 = (int64_t)n_mem * T * d_v / 4;
  const int64_t cb = (n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192;
  const f32x4* const part = reinterpret_cast<const f32x4*>(base + L.part);
  f32x4* const o4 = reinterpret_cast<f32x4*>(out);
  if (S == 2)
    hipLaunchKernelGGL(combine_kernel<2>, dim3((unsigned)cb), dim3(256), 0, stream, part, o4, n4);
  else
    hipLaunchKernelGGL(combine_kernel<8>, dim3((unsigned)cb), dim3(256), 0, stream, part, o4, n4);
  return hipGetLastError();
}

}  // namespace sdm
