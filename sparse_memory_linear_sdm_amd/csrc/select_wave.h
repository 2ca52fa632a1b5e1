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
//            largest key is found by bisection on the key value, counting
//            with ballots; the search stops as soon as a probe threshold has
//            exactly K keys at or above it.  Ties at the final threshold are
//            resolved by a second bisection on the index.
//   stage 2  the K stage-1 survivors of x2 are bitonic-sorted (one per lane).
//            Lane i owns candidate row i (value x1[A_i]); for any threshold
//            t the row's candidates with key(fl(x1[A_i] + x2[B_j])) >= t form
//            a prefix j < L_i(t) of the sorted B, because binary32 addition
//            is monotone.  Bisection on t with counts sum_i L_i(t) (each L_i
//            found by a per-lane binary search inside the bracket left by
//            the previous probe) gives the K best candidates, again with a
//            second bisection on f for ties.  Only those K are sorted.
//   weights  softmax of the K selected sums in fp32 (expf).
#pragma once
#include "device_common.h"

namespace sdm {

struct SelectLds {
  uint32_t akey[64];  // stage-1 survivors of x1: key, index
  int32_t aidx[64];
  uint32_t bkey[64];  // stage-1 survivors of x2, sorted by (key desc, idx asc)
  int32_t bidx[64];
  uint64_t cand[64];  // stage-2 survivors: (key << 32) | ~f
};

// Index of register slot p of a lane: groups of 4 consecutive elements per
// lane (float4 loads) when P is a multiple of 4, else one element per lane.
template <int P>
__device__ __forceinline__ int elem_index(int p, int lane) {
  if constexpr (P % 4 == 0) return (p >> 2) * 256 + lane * 4 + (p & 3);
  else return p * 64 + lane;
}

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

template <int P>
__device__ __forceinline__ int count_ge(const uint32_t (&u)[P], uint32_t t, int n, int lane) {
  int c = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    bool valid = (P > 1) || (lane < n);
    c += __popcll(__ballot(valid && u[p] >= t));
  }
  return c;
}

// Stage 1 for one half: writes the K survivors (key, index) to LDS in index
// order of their register slots (not sorted).
template <int P>
__device__ __forceinline__ void stage1(const uint32_t (&u)[P], int n, int K, int lane,
                                       uint32_t* out_key, int32_t* out_idx) {
  const bool full = (P > 1) || (n >= 64);
  uint32_t lmax = 0, lmin = 0xFFFFFFFFu;
  bool any = false;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    bool valid = (P > 1) || (lane < n);
    if (valid) {
      lmax = u[p] > lmax ? u[p] : lmax;
      lmin = u[p] < lmin ? u[p] : lmin;
      any = true;
    }
  }
  uint64_t hi = (uint64_t)wave_max_u32(any ? lmax : 0u) + 1;
  // Every lane holds at least one key when the wave is full, so the smallest
  // lane maximum has >= 64 >= K keys at or above it.
  uint64_t lo = full ? (uint64_t)wave_min_u32(lmax) : (uint64_t)wave_min_u32(lmin);
  int clo = count_ge<P>(u, (uint32_t)lo, n, lane);
  bool exact = (clo == K);
  while (!exact && hi - lo > 1) {
    uint64_t mid = lo + ((hi - lo) >> 1);
    int c = count_ge<P>(u, (uint32_t)mid, n, lane);
    if (c == K) {
      lo = mid;
      exact = true;
    } else if (c > K) {
      lo = mid;
    } else {
      hi = mid;
    }
  }
  const uint32_t tau = (uint32_t)lo;
  // Tie handling: keys > tau all go in; m = K - #(> tau) of the keys == tau
  // with the lowest indices go in.  ibound = first index NOT taken.
  int ibound = 0x7FFFFFFF;
  if (!exact) {
    int cgt = count_ge<P>(u, tau + 1u, n, lane);  // tau < 0xFFFFFFFF here
    int m = K - cgt;
    int ilo = 0, ihi = n;  // smallest ibound with #(== tau, idx < ibound) >= m
    while (ilo < ihi) {
      int mid = (ilo + ihi) >> 1;
      int c = 0;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        bool valid = (P > 1) || (lane < n);
        c += __popcll(__ballot(valid && u[p] == tau && elem_index<P>(p, lane) < mid + 1));
      }
      if (c >= m) ihi = mid;
      else ilo = mid + 1;
    }
    ibound = ilo + 1;
  }
  int base = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int p = 0; p < P; ++p) {
    bool valid = (P > 1) || (lane < n);
    int i = elem_index<P>(p, lane);
    bool sel = valid && (exact ? (u[p] >= tau)
                               : (u[p] > tau || (u[p] == tau && i < ibound)));
    uint64_t mask = __ballot(sel);
    if (sel) {
      int pos = base + __popcll(mask & below);
      out_key[pos] = u[p];
      out_idx[pos] = i;
    }
    base += __popcll(mask);
  }
}

// Number of j in [l, r) (prefix property) with key(a + B_j) >= t, returned as
// the prefix end.
__device__ __forceinline__ int prefix_end(float a, const uint32_t* bkey, int l, int r,
                                          uint32_t t) {
  while (l < r) {
    int m = (l + r) >> 1;
    if (okey(a + okey_inv(bkey[m])) >= t) l = m + 1;
    else r = m;
  }
  return l;
}

// Full selection of one unit.  x1, x2 point at this unit's n values.
// Writes K outputs per unit (lanes j < K write slot j).
template <int P>
__device__ void select_unit(const float* __restrict__ x1, const float* __restrict__ x2, int n,
                            int K, SelectLds& s, int32_t* __restrict__ idx_out,
                            float* __restrict__ score_out, float* __restrict__ weight_out) {
  const int lane = lane_id();
  uint32_t u[P];

  // ---- stage 1, both halves
  load_keys<P>(x1, n, lane, u);
  stage1<P>(u, n, K, lane, s.akey, s.aidx);
  load_keys<P>(x2, n, lane, u);
  stage1<P>(u, n, K, lane, s.bkey, s.bidx);
  wave_sync();

  // ---- sort B survivors by (key desc, index asc)
  {
    uint64_t kb = 0;
    if (lane < K) kb = ((uint64_t)s.bkey[lane] << 32) | (uint32_t)(~(uint32_t)s.bidx[lane]);
    kb = wave_sort_desc_u64(kb);
    wave_sync();
    if (lane < K) {
      s.bkey[lane] = (uint32_t)(kb >> 32);
      s.bidx[lane] = (int32_t)(~(uint32_t)kb);
    }
    wave_sync();
  }

  // ---- stage 2: lane i owns candidate row A_i
  const bool row = lane < K;
  const float a = row ? okey_inv(s.akey[lane]) : 0.0f;
  const int32_t arow = row ? s.aidx[lane] : 0;
  const float amax = okey_inv(wave_max_u32(row ? s.akey[lane] : 0u));
  const float b0 = okey_inv(s.bkey[0]);
  const float bl = okey_inv(s.bkey[K - 1]);
  uint64_t lo = okey(amax + bl);            // the row of amax has K candidates >= lo
  uint64_t hi = (uint64_t)okey(amax + b0) + 1;  // no candidate reaches hi
  int Llo = 0;                              // L_i(hi)
  int Lhi = row ? prefix_end(a, s.bkey, 0, K, (uint32_t)lo) : 0;  // L_i(lo)
  bool exact = (wave_sum_i32(Lhi) == K);
  int Lsel = Lhi;
  while (!exact && hi - lo > 1) {
    uint64_t mid = lo + ((hi - lo) >> 1);
    int L = row ? prefix_end(a, s.bkey, Llo, Lhi, (uint32_t)mid) : 0;
    int c = wave_sum_i32(L);
    if (c == K) {
      exact = true;
      Lsel = L;
    } else if (c > K) {
      lo = mid;
      Lhi = L;
    } else {
      hi = mid;
      Llo = L;
    }
  }
  // Selected candidates of this lane's row: j < Lsel (exact case), or
  // j < Llo plus the ties j in [Llo, Lhi) (all with key == lo) whose flat
  // index is below fbound.
  int fbound = 0;
  if (!exact) {
    int cgt = wave_sum_i32(Llo);
    int m = K - cgt;
    const int nn = n * n;
    int flo = 0, fhi = nn;  // smallest fb with #(ties with f < fb) >= m
    while (flo < fhi) {
      int fm = flo + ((fhi - flo) >> 1);
      int c = 0;
      if (row)
        for (int j = Llo; j < Lhi; ++j) c += (arow * n + s.bidx[j] < fm + 1) ? 1 : 0;
      c = wave_sum_i32(c);
      if (c >= m) fhi = fm;
      else flo = fm + 1;
    }
    fbound = flo + 1;
  }
  // Compact the K selected candidates into LDS.
  {
    int cnt = 0;
    if (row) {
      if (exact) cnt = Lsel;
      else {
        cnt = Llo;
        for (int j = Llo; j < Lhi; ++j) cnt += (arow * n + s.bidx[j] < fbound) ? 1 : 0;
      }
    }
    int pos = wave_excl_scan_i32(cnt);
    if (row) {
      int end = exact ? Lsel : Lhi;
      for (int j = 0; j < end; ++j) {
        int32_t f = arow * n + s.bidx[j];
        if (!exact && j >= Llo && f >= fbound) continue;
        float sig = a + okey_inv(s.bkey[j]);
        s.cand[pos++] = ((uint64_t)okey(sig) << 32) | (uint32_t)(~(uint32_t)f);
      }
    }
    wave_sync();
  }

  // ---- order the K outputs and form the softmax weights
  uint64_t kc = lane < K ? s.cand[lane] : 0ull;
  kc = wave_sort_desc_u64(kc);
  const float sig = okey_inv((uint32_t)(kc >> 32));
  const float top = __shfl(sig, 0);
  const float e = lane < K ? expf(sig - top) : 0.0f;
  const float z = wave_sum_f32(e);
  if (lane < K) {
    idx_out[lane] = (int32_t)(~(uint32_t)kc);
    if (score_out) score_out[lane] = sig;
    weight_out[lane] = e / z;
  }
  wave_sync();
}

}  // namespace sdm
