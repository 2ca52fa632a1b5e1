// Product-key top-K selection by one wavefront (page "Riepilogo Tecnico:
// Sparse Delta Memory (SDM)", section "Meccanismo Core", item 2: the top-K
// of the N = n*n sums x1[a] + x2[b] is taken as topk(topk(x1) (+) topk(x2))).
//
// Exact orders (the result is unique):
//   stage 1: value descending, index ascending on equal values;
//   stage 2: binary32 sum descending, flat index f = a*n + b ascending.
//
// Method, per unit, on one wave of 64 lanes and no sorting of the inputs:
//   stage 1  each lane holds P = n/64 order-preserving uint32 keys.  The K-th
//            largest key is found either by bisection on the key value (each
//            probe counts in registers and sums over the wave; the search
//            stops as soon as a probe has exactly K keys at or above it), or
//            by a radix search over the key range [lo, hi): the keys in range
//            are counted into a 256-bin LDS histogram by the top 8 bits of
//            key - lo, one suffix scan over the bins finds the bin holding
//            the K-th largest, and the range shrinks to that bin (at most four
//            passes; it stops as soon as a bin holds exactly the keys still
//            needed).  Ties at the final threshold are resolved by bisection
//            on the index.
//   stage 2  both survivor lists are sorted (rank r for x1, c for x2).  With
//            both sorted, key(r, c) = key(fl(A_r + B_c)) does not increase
//            along a row or a column (binary32 addition is monotone), so the
//            set {key >= t} is a staircase.  A staircase holding at least K
//            candidates holds at least K of the set
//                P+ = {(r, c) : (r+1)(c+1) <= K}
//                     plus, per row, the first pair past that bound,
//            and one holding exactly K of P+ lies inside P+ (a staircase that
//            leaves P+ contains a row prefix reaching past the bound, which
//            already holds K pairs of P+, plus that row's boundary pair).
//            P+ has at most 343 pairs for K <= 64, so every lane keeps <= 6
//            of their keys in registers and the search of stage 1 applies to
//            P+ unchanged.  Ties at the K-th key are broken by bisection
//            on f.  Ties only extend past P+ through a boundary pair; in that
//            rare case the affected rows' tied runs are added from LDS.
//   weights  softmax of the K selected sums in fp32 (expf).
#pragma once
#include "device_common.h"

namespace sdm {

// ---- the pair lists P+ for every K in 1..64, row-major, entry (r << 8) | c
namespace pairtab {
constexpr int kMaxK = 64;
constexpr int kSlots = 6;  // ceil(max over K of |P+| / 64)
constexpr int row_len(int K, int r) { return K / (r + 1) + 1 < K ? K / (r + 1) + 1 : K; }
constexpr int list_len(int K) {
  int s = 0;
  for (int r = 0; r < K; ++r) s += row_len(K, r);
  return s;
}
constexpr int total_len() {
  int s = 0;
  for (int K = 1; K <= kMaxK; ++K) s += list_len(K);
  return s;
}
constexpr int kTotal = total_len();
struct Table {
  uint16_t start[kMaxK + 1];
  uint16_t len[kMaxK + 1];
  uint16_t rc[kTotal];
};
constexpr Table make() {
  Table t{};
  int o = 0;
  for (int K = 1; K <= kMaxK; ++K) {
    t.start[K] = (uint16_t)o;
    t.len[K] = (uint16_t)list_len(K);
    for (int r = 0; r < K; ++r)
      for (int c = 0; c < row_len(K, r); ++c) t.rc[o++] = (uint16_t)((r << 8) | c);
  }
  return t;
}
static_assert(list_len(kMaxK) <= kSlots * 64, "slot count");
}  // namespace pairtab

static __constant__ const pairtab::Table kPairTab = pairtab::make();

struct SelectLds {
  // The survivors of each half as 64-bit words (key << 32) | ~index: stage 1
  // writes them in no particular order; select_finish sorts them in place,
  // or sort_survivors does, on the wave that wrote the half.
  struct {
    uint64_t a[64];
    uint64_t b[64];
  } sorted;
  uint64_t cand[64];   // the K selected: (key << 32) | ~f
  uint64_t trash[64];  // per-lane sink of stage 1's branch-free compaction
  alignas(16) uint32_t hist[256];  // radix-search histogram of the wave that owns this
};

// Index of register slot p of a lane: groups of 4 consecutive elements per
// lane (float4 loads) when P is a multiple of 4, else one element per lane.
template <int P>
__device__ __forceinline__ int elem_index(int p, int lane) {
  if constexpr (P % 4 == 0) return (p >> 2) * 256 + lane * 4 + (p & 3);
  else return p * 64 + lane;
}

// Keys of one half; slots past n hold 0, below every key of a finite value
// (those are >= 0x007FFFFF).
template <int P>
__device__ __forceinline__ void load_keys(const float* __restrict__ x, int n, int lane,
                                          uint32_t (&u)[P]) {
  if constexpr (P % 4 == 0) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
#pragma unroll
    for (int q = 0; q < P / 4; ++q) {
      f32x4 f = __builtin_nontemporal_load(x4 + q * 64 + lane);
      u[4 * q + 0] = okey(f.x);
      u[4 * q + 1] = okey(f.y);
      u[4 * q + 2] = okey(f.z);
      u[4 * q + 3] = okey(f.w);
    }
  } else {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      int i = p * 64 + lane;
      u[p] = i < n ? okey(x[i]) : 0u;
    }
  }
}

// Number of keys >= t over the wave (wave-uniform).  Every threshold used is
// >= 1, so slots holding 0 never count.
template <int P>
__device__ __forceinline__ int count_ge(const uint32_t (&u)[P], uint32_t t) {
  // one vector compare per key into a scalar mask, four masks live at a time
  // (independent scalar registers), popcounts and adds on the scalar unit
  int c = 0;
#pragma unroll
  for (int p = 0; p < P; p += 4) {
    uint64_t b[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (p + q < P) b[q] = __ballot(u[p + q] >= t);
    c += (__popcll(b[0]) + __popcll(b[1])) + (__popcll(b[2]) + __popcll(b[3]));
  }
  return c;
}

// Bisection for the K-th largest of the wave's keys, from lo with
// count(>= lo) >= K and hi with count(>= hi) < K.  Returns the threshold;
// *exact tells whether exactly K keys are >= it (else it is the K-th key
// itself, held by more than one key, and ties at it must be broken).
template <int P>
__device__ __forceinline__ uint32_t kth_key_bisect(const uint32_t (&u)[P], int K, uint64_t lo, uint64_t hi,
                                            bool* exact_out) {
  bool exact = count_ge<P>(u, (uint32_t)lo) == K;
  while (!exact && hi - lo > 1) {
    const uint64_t mid = lo + ((hi - lo) >> 1);
    const int c = count_ge<P>(u, (uint32_t)mid);
    if (c >= K) {
      lo = mid;
      exact = (c == K);
    } else {
      hi = mid;
    }
  }
  *exact_out = exact;
  return (uint32_t)lo;
}

// The same result by a radix search, in [lo, hi) where
// count(>= lo) >= K and count(>= hi) < K.  Each pass counts the keys in
// range into a 256-bin histogram (LDS, one per wave) by the top 8 bits of
// key - lo, finds the bin d* holding the K-th largest with one suffix scan
// over the bins (lane l holds bins 4l .. 4l+3), and continues inside that
// bin.  Returns the threshold; *exact tells whether exactly K keys are >= it
// (else it is the K-th key itself, held by more than one key, and ties at it
// must be broken).  Fewer dependent steps than the bisection (at most four
// passes of a few LDS round trips, against 15-30 probes) but, over the n/64
// keys per lane of stage 1, more instructions: the fused decode step (one
// unit per wave, latency-bound) uses it in both stages; the batched
// selection (throughput-bound) in stage 2 only, where each lane holds at most
// six candidate keys (measured: stage 1 by bisection and stage 2 by this
// search is the fastest of the four combinations there).
template <int P>
__device__ __forceinline__ uint32_t kth_key_radix(const uint32_t (&u)[P], int K, uint64_t lo,
                                                  uint64_t hi, bool* exact_out, uint32_t* hist) {
  const int lane = lane_id();
  int krem = K - (hi > 0xFFFFFFFFull ? 0 : count_ge<P>(u, (uint32_t)hi));  // still needed in range
  for (;;) {
    const uint64_t range = hi - lo;  // >= 1
    const int bits = range > 1 ? 64 - __builtin_clzll(range - 1) : 0;
    const int shift = bits > 8 ? bits - 8 : 0;
    const uint32_t lo32 = (uint32_t)lo;
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_sync();
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (u[p] >= lo && (uint64_t)u[p] < hi) atomicAdd(&hist[(u[p] - lo32) >> shift], 1u);
    wave_sync();
    const uint4 b = reinterpret_cast<const uint4*>(hist)[lane];
    const int local = (int)(b.x + b.y + b.z + b.w);
    const int excl = wave_excl_scan_i32(local);
    const int total = __builtin_amdgcn_readlane(excl + local, 63);
    const int g4 = total - excl - local;  // keys in the bins of higher lanes
    const int g3 = g4 + (int)b.w, g2 = g3 + (int)b.z, g1 = g2 + (int)b.y, g0 = g1 + (int)b.x;
    // d* = 4l + j with count(digit >= d*) >= krem > count(digit > d*): one lane, one j
    int j = -1, gt = 0, bc = 0;
    if (g3 >= krem && g4 < krem) { j = 3; gt = g4; bc = (int)b.w; }
    else if (g2 >= krem && g3 < krem) { j = 2; gt = g3; bc = (int)b.z; }
    else if (g1 >= krem && g2 < krem) { j = 1; gt = g2; bc = (int)b.y; }
    else if (g0 >= krem && g1 < krem) { j = 0; gt = g1; bc = (int)b.x; }
    const int L = __ffsll((unsigned long long)__ballot(j >= 0)) - 1;
    const int dstar = 4 * L + __builtin_amdgcn_readlane(j, L);
    krem -= __builtin_amdgcn_readlane(gt, L);
    const int bcount = __builtin_amdgcn_readlane(bc, L);
    const uint64_t nlo = lo + ((uint64_t)dstar << shift);
    const uint64_t nhi = nlo + (1ull << shift) < hi ? nlo + (1ull << shift) : hi;
    wave_sync();  // the histogram is cleared again by the next pass
    if (bcount == krem) {  // every key of the bin goes in: the bin's smallest key is the threshold
      uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
      for (int p = 0; p < P; ++p) mn = (u[p] >= nlo && (uint64_t)u[p] < nhi && u[p] < mn) ? u[p] : mn;
      *exact_out = true;
      return wave_min_u32(mn);
    }
    if (shift == 0) {  // the bin is one key value, held by more keys than still needed
      *exact_out = false;
      return (uint32_t)nlo;
    }
    lo = nlo;
    hi = nhi;
  }
}

// Stage 1 for one half: writes the K survivors to LDS as (key << 32) | ~index,
// in no particular order.  Every slot is stored; a slot that is not selected
// goes to the lane's own trash word, so the compaction has no branches.
template <int P, bool RADIX>
__device__ __forceinline__ void stage1(const uint32_t (&u)[P], int n, int K, int lane,
                                       uint64_t* out, uint64_t* trash, uint32_t* hist) {
  uint32_t lmax = 0, lmin = 0xFFFFFFFFu;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    lmax = u[p] > lmax ? u[p] : lmax;
    lmin = (u[p] != 0u && u[p] < lmin) ? u[p] : lmin;
  }
  const uint64_t hi = (uint64_t)wave_max_u32(lmax) + 1;
  // With n >= 64 every lane holds a key, so the smallest lane maximum has
  // >= 64 >= K keys at or above it; otherwise start from the smallest key.
  const uint64_t lo = (n >= 64) ? (uint64_t)wave_min_u32(lmax) : (uint64_t)wave_min_u32(lmin);
  bool exact;
  const uint32_t tau = RADIX ? kth_key_radix<P>(u, K, lo, hi, &exact, hist)
                             : kth_key_bisect<P>(u, K, lo, hi, &exact);
  // Tie handling: keys > tau all go in; m = K - #(> tau) of the keys == tau
  // with the lowest indices go in.  ibound = first index NOT taken.
  int ibound = 0x7FFFFFFF;
  if (!exact) {
    const int m = K - count_ge<P>(u, tau + 1u);  // keys of finite values stay below 0xFFFFFFFF
    int ilo = 1, ihi = n;  // smallest ib with #(== tau, idx < ib) >= m
    while (ilo < ihi) {
      const int mid = (ilo + ihi) >> 1;
      int c = 0;
#pragma unroll
      for (int p = 0; p < P; ++p) c += (u[p] == tau && elem_index<P>(p, lane) < mid) ? 1 : 0;
      if (wave_sum_i32(c) >= m) ihi = mid;
      else ilo = mid + 1;
    }
    ibound = ilo;
  }
  bool sel[P];
#pragma unroll
  for (int p = 0; p < P; ++p)  // exactly K keys >= tau (the usual case), else ties cut at ibound
    sel[p] = exact ? u[p] >= tau
                   : (u[p] > tau || (u[p] == tau && elem_index<P>(p, lane) < ibound));
  int cnt = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) cnt += sel[p] ? 1 : 0;
  int pos = wave_excl_scan_i32(cnt);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const uint32_t i = (uint32_t)elem_index<P>(p, lane);
    uint64_t* const d = sel[p] ? out + pos : trash + lane;
    *d = ((uint64_t)u[p] << 32) | (uint32_t)~i;
    pos += sel[p] ? 1 : 0;
  }
}

__device__ __forceinline__ float sorted_val(uint64_t w) { return okey_inv((uint32_t)(w >> 32)); }
__device__ __forceinline__ int32_t sorted_idx(uint64_t w) { return (int32_t)(~(uint32_t)w); }

// Number of c in [l, r) with key(a + B_c) >= t (a prefix of [l, r) by
// monotonicity), returned as the prefix end.
__device__ __forceinline__ int prefix_end(float a, const uint64_t* b, int l, int r, uint32_t t) {
  while (l < r) {
    const int m = (l + r) >> 1;
    if (okey(a + sorted_val(b[m])) >= t) l = m + 1;
    else r = m;
  }
  return l;
}

// Entries of the pair list P+ of this K held by this lane (issued early so
// that their latency hides under stage 1).
__device__ __forceinline__ void pair_slots(int K, uint32_t (&rc)[pairtab::kSlots]) {
  const int lane = lane_id();
  const int plen = kPairTab.len[K];
  const uint16_t* prc = kPairTab.rc + kPairTab.start[K];
#pragma unroll
  for (int p = 0; p < pairtab::kSlots; ++p) {
    const int q = p * 64 + lane;
    rc[p] = q < plen ? prc[q] : 0xFFFFu;
  }
}

// Stage 1 of one half, from its n values in memory to its K survivors in LDS.
template <int P, bool RADIX>
__device__ __forceinline__ void stage1_half(const float* __restrict__ x, int n, int K,
                                            uint64_t* out, uint64_t* trash, uint32_t* hist) {
  uint32_t u[P];
  load_keys<P>(x, n, lane_id(), u);
  stage1<P, RADIX>(u, n, K, lane_id(), out, trash, hist);
}

// One half's K survivors (list[0 .. K)) sorted in place by (key desc, index
// asc); entries K .. 63 become 0, below every survivor word.
__device__ __forceinline__ void sort_survivors(uint64_t* list, int K) {
  const int lane = lane_id();
  uint64_t k = lane < K ? list[lane] : 0ull;
  k = wave_sort_desc_u64(k);
  wave_sync();
  list[lane] = k;
  wave_sync();
}

// Everything after stage 1: both halves' survivors are in s.sorted (written
// by this wave, or by others before a barrier; SORTED: already sorted by
// sort_survivors).  Writes K outputs per unit (lanes j < K write slot j).
template <bool RADIX, bool SORTED = false>
__device__ inline void select_finish(int n, int K, SelectLds& s, const uint32_t (&rc)[pairtab::kSlots],
                              int32_t* __restrict__ idx_out, float* __restrict__ score_out,
                              float* __restrict__ weight_out) {
  constexpr int S = pairtab::kSlots;
  const int lane = lane_id();

  // ---- sort both survivor lists by (key desc, index asc)
  if constexpr (!SORTED) {
    uint64_t ka = lane < K ? s.sorted.a[lane] : 0ull, kb = lane < K ? s.sorted.b[lane] : 0ull;
    wave_sort2_desc_u64(ka, kb);
    wave_sync();
    s.sorted.a[lane] = ka;
    s.sorted.b[lane] = kb;
    wave_sync();
  }

  // ---- stage 2 over P+: slot keys and flat indices in registers
  uint32_t sk[S];
  int32_t sf[S];
  uint32_t bnd = 0;  // bit p: slot p is a boundary pair, (r+1)(c+1) > K
#pragma unroll
  for (int p = 0; p < S; ++p) {
    sk[p] = 0u;
    sf[p] = 0x7FFFFFFF;
    if (rc[p] != 0xFFFFu) {
      const int r = (int)(rc[p] >> 8), c = (int)(rc[p] & 0xFFu);
      const uint64_t wa = s.sorted.a[r], wb = s.sorted.b[c];
      sk[p] = okey(sorted_val(wa) + sorted_val(wb));
      sf[p] = sorted_idx(wa) * n + sorted_idx(wb);
      bnd |= ((r + 1) * (c + 1) > K) ? (1u << p) : 0u;
    }
  }
  const float a0 = sorted_val(s.sorted.a[0]);
  // Row 0 holds K pairs of P+ with key >= key(A_0 + B_{K-1}); none reaches
  // key(A_0 + B_0) + 1.
  const uint64_t lo0 = okey(a0 + sorted_val(s.sorted.b[K - 1]));
  const uint64_t hi0 = (uint64_t)okey(a0 + sorted_val(s.sorted.b[0])) + 1;
  bool exact;
  const uint32_t tau = RADIX ? kth_key_radix<S>(sk, K, lo0, hi0, &exact, s.hist)
                             : kth_key_bisect<S>(sk, K, lo0, hi0, &exact);

  // Ties at tau (not exact): m of them go in, lowest f first.  Tied pairs
  // outside P+ exist only in rows whose boundary pair ties; lane r then adds
  // the tied columns (cb, xhi) of row r.
  int fbound = 0x7FFFFFFF;
  int xlo = 0, xhi = 0;
  int32_t arow_idx = 0;
  if (!exact) {
    const int m = K - count_ge<S>(sk, tau + 1u);
    bool btie = false;
#pragma unroll
    for (int p = 0; p < S; ++p) btie |= ((bnd >> p) & 1u) && sk[p] == tau;
    if (__ballot(btie) != 0ull && lane < K) {
      const int cb = K / (lane + 1);
      if (cb < K) {
        const uint64_t wa = s.sorted.a[lane];
        const float arow = sorted_val(wa);
        if (okey(arow + sorted_val(s.sorted.b[cb])) == tau) {
          arow_idx = sorted_idx(wa);
          xlo = cb + 1;
          xhi = prefix_end(arow, s.sorted.b, cb + 1, K, tau);
        }
      }
    }
    int flo = 1, fhi = n * n;  // smallest fb with #(ties, f < fb) >= m
    while (flo < fhi) {
      const int fm = flo + ((fhi - flo) >> 1);
      int c = 0;
#pragma unroll
      for (int p = 0; p < S; ++p) c += (sk[p] == tau && sf[p] < fm) ? 1 : 0;
      for (int j = xlo; j < xhi; ++j) c += (arow_idx * n + sorted_idx(s.sorted.b[j]) < fm) ? 1 : 0;
      if (wave_sum_i32(c) >= m) fhi = fm;
      else flo = fm + 1;
    }
    fbound = flo;
  }

  // ---- compact the K selected pairs into LDS
  {
    int cnt = 0;
#pragma unroll
    for (int p = 0; p < S; ++p)
      cnt += (sk[p] > tau || (sk[p] == tau && (exact || sf[p] < fbound))) ? 1 : 0;
    for (int j = xlo; j < xhi; ++j)
      cnt += (arow_idx * n + sorted_idx(s.sorted.b[j]) < fbound) ? 1 : 0;
    int pos = wave_excl_scan_i32(cnt);
#pragma unroll
    for (int p = 0; p < S; ++p) {
      if (sk[p] > tau || (sk[p] == tau && (exact || sf[p] < fbound)))
        s.cand[pos++] = ((uint64_t)sk[p] << 32) | (uint32_t)(~(uint32_t)sf[p]);
    }
    for (int j = xlo; j < xhi; ++j) {
      const int32_t f = arow_idx * n + sorted_idx(s.sorted.b[j]);
      if (f < fbound) s.cand[pos++] = ((uint64_t)tau << 32) | (uint32_t)(~(uint32_t)f);
    }
    wave_sync();
  }

  // ---- order the K outputs and form the softmax weights
  uint64_t kc = lane < K ? s.cand[lane] : 0ull;
  kc = wave_sort_desc_u64(kc);
  const float sig = okey_inv((uint32_t)(kc >> 32));
  const float top = lane0_f32(sig);
  const float e = lane < K ? expf(sig - top) : 0.0f;
  const float z = wave_sum_f32(e);
  if (lane < K) {
    idx_out[lane] = (int32_t)(~(uint32_t)kc);
    if (score_out) score_out[lane] = sig;
    weight_out[lane] = e / z;
  }
  wave_sync();
}

// Full selection of one unit by one wave.  x1, x2 point at this unit's n
// values.
template <int P>
__device__ void select_unit(const float* __restrict__ x1, const float* __restrict__ x2, int n,
                            int K, SelectLds& s, int32_t* __restrict__ idx_out,
                            float* __restrict__ score_out, float* __restrict__ weight_out) {
  uint32_t rc[pairtab::kSlots];
  pair_slots(K, rc);
  stage1_half<P, false>(x1, n, K, s.sorted.a, s.trash, s.hist);
  stage1_half<P, false>(x2, n, K, s.sorted.b, s.trash, s.hist);
  wave_sync();
  select_finish<true>(n, K, s, rc, idx_out, score_out, weight_out);
}

}  // namespace sdm
