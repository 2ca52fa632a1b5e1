// Reverse pass of the SDM step for training: gradients of the gated delta
// write and the sparse read (page "Riepilogo Tecnico: Sparse Delta Memory
// (SDM)", section "Meccanismo Core", items 3 and 4) with the selections held
// fixed, the selection weights' gradient taken back to the key halves
// (item 2: slot a*n + b scores x1[a] + x2[b]), and the gradient of the
// learned initial state (section "Stato Iniziale Appreso").
//
// Per step, for write row i = f_j with pre-write stored row P and
// g = dL/dM_t[i] (this step's read part included):
//   u = alpha*(1 - beta*k_j)*P + beta*k_j*v          (the forward write)
//   dv += beta*k_j*g;  dalpha += (1 - beta*k_j)*<g, P>;
//   d(beta*k_j) = <g, v - alpha*P>;  dM_{t-1}[i] = alpha*(1 - beta*k_j)*g
// and for read row g_j: dr_j = <do, M_t[g_j]>, dM_t[g_j] += r_j*do.
// Rows that a step does not write carry their gradient unchanged.
//
// scan_bwd_kernel walks t = T-1 .. 0 with one wavefront per (memory,
// column tile: 32 columns, or 16 in the sparse mode).  The training forward kept a tape of each step's W
// pre-write rows and R read rows (the values the read used), so this pass
// never touches the state M: every value it needs is on the tape, stored
// contiguously per step.  The gradient table G (caller-owned, the shape of
// M) starts as dL/dM_T and ends as dL/dM_0.  Each step gathers the read and
// the write rows of G (16-byte buffer loads of one tile row per lane group)
// and its tape rows, matches write rows against this step's read rows
// through a hashed LDS table, and stores G's read rows, then G's write rows
// -- in that order, so a row that is both read and written ends with its
// write-side value.  All accesses to a (row, tile) of G come from one
// wavefront, and the next step's loads are issued after this step's stores,
// so program order keeps every step's view current.  Per-tile partial sums
// of d(beta*k), dr and dalpha go to a caller-provided workspace; a
// finishing kernel adds the tiles in a fixed order (deterministic) and
// applies beta and the k weights.
//
// Sparse mode (the final-state gradient is zero): touch_kernel marks, per
// step, the slots whose row the forward selects there for the last time;
// the reverse scan gathers no G for them (zero, as a cleared table would
// give), so G is never cleared, and the M0 gradient reads only the rows a
// sequence selects.  Nothing here is a dense contraction: no MFMA.
#include "device_common.h"
#include "internal.h"
#include "ranges.h"

namespace sdm {
namespace {

constexpr int kBufWord3 = 0x00020000;  // raw buffer access, gfx9 family
constexpr uint32_t kOffNone = ranges::kOffNone;  // outside every range: loads 0, stores dropped
constexpr int kHashBits = 12;

struct BwdArgs {
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
  const float* dout;
  const float* tape;
  float* G;
  float* dv;
  float* ws;
  int ntiles;
  const uint64_t* first;  // optional: per step, the slots that are their row's last touch
};

__device__ __forceinline__ uint32_t hash_slot(uint32_t row) {
  return (row * 2654435761u) >> (32 - kHashBits);
}

__device__ __forceinline__ f32x4 as_f4(const u32x4& q) {
  return f32x4{__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
               __uint_as_float(q.w)};
}
__device__ __forceinline__ u32x4 as_u4(const f32x4& f) {
  return u32x4{__float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(f.z),
               __float_as_uint(f.w)};
}

template <int O>
__device__ __forceinline__ float xor_add(float x) {
  return x + __uint_as_float(lane_xor(__float_as_uint(x), O));
}

// Sum over the LPR lanes that hold one row (lanes differ in the low bits).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR >= 2) x = xor_add<1>(x);
  if constexpr (LPR >= 4) x = xor_add<2>(x);
  if constexpr (LPR >= 8) x = xor_add<4>(x);
  return x;
}

// Sum over the lanes that hold the same columns (lanes differ in the high bits).
template <int LPR>
__device__ __forceinline__ float col_sum(float x) {
  if constexpr (LPR <= 4) x = xor_add<4>(x);
  if constexpr (LPR <= 8) x = xor_add<8>(x);
  x = xor_add<16>(x);
  x = xor_add<32>(x);
  return x;
}

template <int COLS>
__global__ __launch_bounds__(kWave) void scan_bwd_kernel(BwdArgs A) {
  constexpr int LPR = COLS / 4;      // lanes per tile row (16 bytes each)
  constexpr int RPI = kWave / LPR;   // rows per wave instruction
  constexpr int NI = 64 / RPI;       // instructions for 64 row slots
  __shared__ uint64_t tab[1 << kHashBits];  // (row << 32) | (t << 6 | slot)
  __shared__ float rws[64];

  // XCD-aware numbering as in the forward: every tile of a memory on one XCD.
  const int bid = blockIdx.x;
  const int x = bid & 7;
  const int rest = bid >> 3;
  const int tile = rest % A.ntiles;
  const int mem = (rest / A.ntiles) * 8 + x;
  if (mem >= A.n_mem) return;

  const int lane = lane_id();
  const int lr = lane / LPR, lc = lane % LPR;
  const int d_v = A.d_v, W = A.W, R = A.R;
  const int64_t T = A.T, N = A.N;
  for (int i = lane; i < (1 << kHashBits); i += kWave) tab[i] = ~0ull;

  // descriptor ranges from ranges.h (checked on the host before the launch)
  const int64_t mem_elems = N * d_v;
  const __amdgpu_buffer_rsrc_t gres = __builtin_amdgcn_make_buffer_rsrc(
      A.G + (int64_t)mem * mem_elems + tile * COLS, 0,
      (int)ranges::table_range(N, (int64_t)d_v * 4, tile, COLS * 4), kBufWord3);
  const int64_t tape_rows = T * (W + R);  // per step: W pre-write rows, R read rows
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(A.tape) + (int64_t)mem * tape_rows * d_v + tile * COLS, 0,
      (int)ranges::table_range(tape_rows, (int64_t)d_v * 4, tile, COLS * 4), kBufWord3);
  const uint32_t row_bytes = (uint32_t)d_v * 4u;
  const uint32_t lane_off = (uint32_t)lc * 16u;

  const int32_t* widx = A.widx + (int64_t)mem * T * W;
  const float* wk = A.wk + (int64_t)mem * T * W;
  const int32_t* ridx = A.ridx + (int64_t)mem * T * R;
  const float* rw = A.rw + (int64_t)mem * T * R;
  const float* vm = A.v + (int64_t)mem * T * d_v + tile * COLS + lc * 4;
  const float* dom = A.dout + (int64_t)mem * T * d_v + tile * COLS + lc * 4;
  float* dvm = A.dv + (int64_t)mem * T * d_v + tile * COLS + lc * 4;
  const float* am = A.alpha + (int64_t)mem * T;
  const float* bm = A.beta + (int64_t)mem * T;
  const int ws_row = W + R + 1;
  float* wsm = A.ws + ((int64_t)mem * T * A.ntiles + tile) * ws_row;
  wave_sync();

  // Step metadata travels one step ahead: during step t the lanes load step
  // t-1's indices, weights, values and gates in "lane j = slot j" layout;
  // after step t they pass through LDS into the per-row layout the gathers
  // use, so a step's gathers are issued without waiting on its metadata.
  __shared__ int32_t sm_w[64], sm_r[64];
  __shared__ float sm_wk[64], sm_rw[64];
  __shared__ f32x4 sm_v[LPR], sm_d[LPR];
  int32_t fw_[NI], fr_[NI];
  float wkk[NI], rwk[NI];
  f32x4 vv, dd;
  float a, b;
  int32_t my_r;
  float my_rw;
  {  // step T-1 directly
    const int64_t t = T - 1;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int j = k * RPI + lr;
      fw_[k] = j < W ? widx[t * W + j] : -1;
      fr_[k] = j < R ? ridx[t * R + j] : -1;
      wkk[k] = j < W ? wk[t * W + j] : 0.0f;
      rwk[k] = j < R ? rw[t * R + j] : 0.0f;
    }
    vv = *reinterpret_cast<const f32x4*>(vm + t * d_v);
    dd = *reinterpret_cast<const f32x4*>(dom + t * d_v);
    a = am[t];
    b = bm[t];
    my_r = lane < R ? ridx[t * R + lane] : -1;
    my_rw = lane < R ? rw[t * R + lane] : 0.0f;
  }
  // Sparse mode: a slot whose row the forward touches for the last time at
  // this step is the row's first touch in reverse, where G holds dL/dM_T =
  // 0 for it; its G gather is dropped (an out-of-range buffer load returns
  // zero), so G needs no zeroing beforehand.
  const uint64_t* firstm = A.first ? A.first + (int64_t)mem * T * 2 : nullptr;
  uint64_t fm_w = firstm ? firstm[(T - 1) * 2] : 0ull, fm_r = firstm ? firstm[(T - 1) * 2 + 1] : 0ull;

  for (int64_t t = T - 1; t >= 0; --t) {
    // ---- this step's offsets
    uint32_t wrow[NI], wo[NI], ro[NI], to[NI], tr[NI], wlo[NI], rlo[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int j = k * RPI + lr;
      const bool wv = (uint32_t)fw_[k] < (uint32_t)N, rv = (uint32_t)fr_[k] < (uint32_t)N;
      wrow[k] = wv ? (uint32_t)fw_[k] : 0xFFFFFFFFu;
      wo[k] = wv ? (uint32_t)fw_[k] * row_bytes + lane_off : kOffNone;
      ro[k] = rv ? (uint32_t)fr_[k] * row_bytes + lane_off : kOffNone;
      const uint32_t tstep = (uint32_t)t * (uint32_t)(W + R);
      to[k] = wv ? (tstep + (uint32_t)j) * row_bytes + lane_off : kOffNone;
      tr[k] = rv ? (tstep + (uint32_t)(W + j)) * row_bytes + lane_off : kOffNone;
      wlo[k] = ((fm_w >> j) & 1ull) ? kOffNone : wo[k];  // G gathers (stores keep wo, ro)
      rlo[k] = ((fm_r >> j) & 1ull) ? kOffNone : ro[k];
    }

    // ---- gathers (all issued before any is used)
    u32x4 Mg[NI], Gg[NI], Gf[NI], P[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) Mg[k] = __builtin_amdgcn_raw_buffer_load_b128(tres, tr[k], 0, 0);
#pragma unroll
    for (int k = 0; k < NI; ++k) Gg[k] = __builtin_amdgcn_raw_buffer_load_b128(gres, rlo[k], 0, 0);
#pragma unroll
    for (int k = 0; k < NI; ++k) Gf[k] = __builtin_amdgcn_raw_buffer_load_b128(gres, wlo[k], 0, 0);
#pragma unroll
    for (int k = 0; k < NI; ++k) P[k] = __builtin_amdgcn_raw_buffer_load_b128(tres, to[k], 0, 0);

    // ---- step t-1's metadata, in flight with the gathers
    const int64_t tn = t > 0 ? t - 1 : 0;
    const int32_t n_w = lane < W ? widx[tn * W + lane] : -1;
    const float n_wk = lane < W ? wk[tn * W + lane] : 0.0f;
    const int32_t n_r = lane < R ? ridx[tn * R + lane] : -1;
    const float n_rw = lane < R ? rw[tn * R + lane] : 0.0f;
    const int lv = lane < LPR ? lane : 0;
    const f32x4 n_v = *reinterpret_cast<const f32x4*>(vm - lc * 4 + lv * 4 + tn * d_v);
    const f32x4 n_d = *reinterpret_cast<const f32x4*>(dom - lc * 4 + lv * 4 + tn * d_v);
    const float n_a = am[tn], n_b = bm[tn];
    const uint64_t n_fw = firstm ? firstm[tn * 2] : 0ull, n_fr = firstm ? firstm[tn * 2 + 1] : 0ull;

    // ---- match write rows to this step's read rows while the gathers fly.
    // Lane j inserts read slot j; a read row whose table entry was taken by
    // another read row of the step (hash collision) is matched by a
    // wave-uniform loop instead.  Entries of other steps carry another stamp.
    const bool my_valid = (uint32_t)my_r < (uint32_t)N;
    const uint32_t stamp = ((uint32_t)t << 6) | (uint32_t)lane;
    const uint64_t entry = ((uint64_t)(uint32_t)my_r << 32) | stamp;
    rws[lane] = my_rw;
    if (my_valid) tab[hash_slot((uint32_t)my_r)] = entry;
    wave_sync();
    const bool lost = my_valid && tab[hash_slot((uint32_t)my_r)] != entry;
    uint64_t lostmask = __ballot(lost);
    int match[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const uint64_t e = tab[hash_slot(wrow[k])];
      const bool hit = wrow[k] != 0xFFFFFFFFu && (uint32_t)(e >> 32) == wrow[k] &&
                       ((uint32_t)e >> 6) == (uint32_t)t;
      match[k] = hit ? (int)(e & 63u) : -1;
    }
    while (lostmask) {
      const int j = __builtin_ctzll(lostmask);
      lostmask &= lostmask - 1;
      const uint32_t s = (uint32_t)__builtin_amdgcn_readlane(my_r, j);
#pragma unroll
      for (int k = 0; k < NI; ++k)
        if (wrow[k] == s) match[k] = j;
    }
    float mw[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) mw[k] = match[k] >= 0 ? rws[match[k]] : 0.0f;

    // ---- read part: dr_j and G[g_j] += r_j * do
    float drp[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const f32x4 m = as_f4(Mg[k]);
      drp[k] = dd.x * m.x + dd.y * m.y + dd.z * m.z + dd.w * m.w;
      f32x4 g = as_f4(Gg[k]);
      g.x = fmaf(rwk[k], dd.x, g.x);
      g.y = fmaf(rwk[k], dd.y, g.y);
      g.z = fmaf(rwk[k], dd.z, g.z);
      g.w = fmaf(rwk[k], dd.w, g.w);
      Gg[k] = as_u4(g);
    }
    // ---- write part
    f32x4 dva = {0.f, 0.f, 0.f, 0.f};
    float dap = 0.0f;
    float dbk[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      f32x4 g = as_f4(Gf[k]);
      g.x = fmaf(mw[k], dd.x, g.x);
      g.y = fmaf(mw[k], dd.y, g.y);
      g.z = fmaf(mw[k], dd.z, g.z);
      g.w = fmaf(mw[k], dd.w, g.w);
      const f32x4 p = as_f4(P[k]);
      const float bk = b * wkk[k];
      dva.x = fmaf(bk, g.x, dva.x);
      dva.y = fmaf(bk, g.y, dva.y);
      dva.z = fmaf(bk, g.z, dva.z);
      dva.w = fmaf(bk, g.w, dva.w);
      const float gp = g.x * p.x + g.y * p.y + g.z * p.z + g.w * p.w;
      dap = fmaf(1.0f - bk, gp, dap);
      dbk[k] = g.x * (vv.x - a * p.x) + g.y * (vv.y - a * p.y) + g.z * (vv.z - a * p.z) +
               g.w * (vv.w - a * p.w);
      const float c = a * (1.0f - bk);
      Gf[k] = as_u4(f32x4{c * g.x, c * g.y, c * g.z, c * g.w});
    }
    // ---- stores: G read rows, then G write rows
#pragma unroll
    for (int k = 0; k < NI; ++k) __builtin_amdgcn_raw_buffer_store_b128(Gg[k], gres, ro[k], 0, 0);
#pragma unroll
    for (int k = 0; k < NI; ++k) __builtin_amdgcn_raw_buffer_store_b128(Gf[k], gres, wo[k], 0, 0);

    // ---- reductions and the step's partial sums
    float* wst = wsm + t * (int64_t)A.ntiles * ws_row;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const float s_bk = row_sum<LPR>(dbk[k]);
      const float s_dr = row_sum<LPR>(drp[k]);
      const int j = k * RPI + lr;
      if (lc == 0) {
        if (j < W) wst[j] = s_bk;
        if (j < R) wst[W + j] = s_dr;
      }
    }
    dva.x = col_sum<LPR>(dva.x);
    dva.y = col_sum<LPR>(dva.y);
    dva.z = col_sum<LPR>(dva.z);
    dva.w = col_sum<LPR>(dva.w);
    if (lr == 0) *reinterpret_cast<f32x4*>(dvm + t * d_v) = dva;
    const float da = wave_sum_f32(dap);
    if (lane == 0) wst[W + R] = da;

    // ---- step t-1's metadata into the per-row layout
    sm_w[lane] = n_w;
    sm_r[lane] = n_r;
    sm_wk[lane] = n_wk;
    sm_rw[lane] = n_rw;
    if (lane < LPR) {
      sm_v[lane] = n_v;
      sm_d[lane] = n_d;
    }
    wave_sync();
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int j = k * RPI + lr;
      fw_[k] = sm_w[j];
      fr_[k] = sm_r[j];
      wkk[k] = sm_wk[j];
      rwk[k] = sm_rw[j];
    }
    vv = sm_v[lc];
    dd = sm_d[lc];
    a = n_a;
    b = n_b;
    fm_w = n_fw;
    fm_r = n_fr;
    my_r = n_r;
    my_rw = n_rw;
    wave_sync();  // the LDS staging, rws and tab are rewritten by the next step
  }
}

// dwk = beta * sum over tiles of d(beta k); drw = sum of dr; dalpha = sum;
// dbeta = sum_j k_j * d(beta k_j).  One wavefront per (memory, step).
__global__ __launch_bounds__(256) void scan_bwd_finish(BwdArgs A, float* __restrict__ dwk,
                                                       float* __restrict__ drw,
                                                       float* __restrict__ dalpha,
                                                       float* __restrict__ dbeta) {
  const int64_t u = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int64_t units = (int64_t)A.n_mem * A.T;
  if (u >= units) return;  // whole wavefront leaves together
  const int lane = lane_id();
  const int W = A.W, R = A.R, ws_row = W + R + 1;
  const float* p = A.ws + u * A.ntiles * ws_row;
  float sbk = 0.0f, sdr = 0.0f, sda = 0.0f;
  for (int tl = 0; tl < A.ntiles; ++tl) {
    const float* q = p + tl * ws_row;
    if (lane < W) sbk += q[lane];
    if (lane < R) sdr += q[W + lane];
    sda += q[W + R];
  }
  const float b = A.beta[u];
  const float kj = lane < W ? A.wk[u * W + lane] : 0.0f;
  if (lane < W) dwk[u * W + lane] = b * sbk;
  if (lane < R) drw[u * R + lane] = sdr;
  const float db = wave_sum_f32(lane < W ? kj * sbk : 0.0f);
  if (lane == 0) {
    dalpha[u] = sda;
    dbeta[u] = db;
  }
}

// Selection weights back to the halves.  One wavefront per unit builds the
// unit's two half-gradient rows in LDS and writes each once: the rows are
// zeroed in LDS, lane j (< K) computes dsigma_j = w_j (dw_j - sum_l w_l dw_l)
// and, for its half indices a_j and b_j, the sum of dsigma_l over every l
// with the same half index (in order l = 0, 1, ...); the lowest such l
// stores it into the LDS row; then the rows go out with coalesced stores.
// (Zeroing the rows in memory and scattering into them wrote 14% more than
// the rows' bytes.)
__global__ __launch_bounds__(256) void select_bwd_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ dw,
                                                         int64_t units, int n, int K,
                                                         float* __restrict__ dx1,
                                                         float* __restrict__ dx2, bool wide) {
  extern __shared__ __align__(16) float rows_lds[];  // [4 waves][2 rows][n]
  const int64_t u = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (u >= units) return;  // whole wavefront leaves together
  const int lane = lane_id();
  float* const l1 = rows_lds + (threadIdx.x / kWave) * 2 * n;
  float* const l2 = l1 + n;
  for (int i = lane; i < n; i += kWave) {
    l1[i] = 0.0f;
    l2[i] = 0.0f;
  }
  const bool on = lane < K;
  const int32_t f = on ? idx[u * K + lane] : 0;
  const float wj = on ? w[u * K + lane] : 0.0f;
  const float dwj = on ? dw[u * K + lane] : 0.0f;
  const float s = wave_sum_f32(wj * dwj);
  const float ds = wj * (dwj - s);
  const int ia = on ? f / n : -1, ib = on ? f % n : -1;
  float sa = 0.0f, sb = 0.0f;
  bool own_a = on, own_b = on;
  for (int l = 0; l < K; ++l) {
    const int al = __builtin_amdgcn_readlane(ia, l);
    const int bl = __builtin_amdgcn_readlane(ib, l);
    const float dl = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(ds), l));
    if (al == ia) {
      sa += dl;
      if (l < lane) own_a = false;
    }
    if (bl == ib) {
      sb += dl;
      if (l < lane) own_b = false;
    }
  }
  wave_sync();
  if (on && (uint32_t)ia < (uint32_t)n && own_a) l1[ia] = sa;
  if (on && (uint32_t)ib < (uint32_t)n && own_b) l2[ib] = sb;
  wave_sync();
  float* const r1 = dx1 + u * n;
  float* const r2 = dx2 + u * n;
  if (wide) {  // n % 4 == 0 and both outputs 16-byte aligned: every row starts aligned
    for (int i = lane; i < n / 4; i += kWave) {
      reinterpret_cast<float4*>(r1)[i] = reinterpret_cast<const float4*>(l1)[i];
      reinterpret_cast<float4*>(r2)[i] = reinterpret_cast<const float4*>(l2)[i];
    }
  } else {
    for (int i = lane; i < n; i += kWave) {
      r1[i] = l1[i];
      r2[i] = l2[i];
    }
  }
}

// dM0[h] = sum over b of G[b, h], in order b = 0, 1, ...  With seen (the
// sparse mode), rows a sequence never selected hold no gradient and are left
// out (their G is not read): adding them as zeros gives the same sum.
template <bool SPARSE>
__global__ __launch_bounds__(256) void init_bwd_kernel(const float4* __restrict__ G,
                                                       float4* __restrict__ dM0, int B,
                                                       int64_t per_seq4, int64_t n4,
                                                       const uint32_t* __restrict__ seen,
                                                       int64_t N, int d4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    float4 acc;
    if constexpr (SPARSE) {
      const int64_t hrow = i / d4;  // h * N + row
      const int64_t H = per_seq4 / d4 / N;
      const int64_t h = hrow / N, row = hrow % N;
      const int64_t words = (N + 31) / 32;
      acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int b = 0; b < B; ++b) {
        if (!((seen[((int64_t)b * H + h) * words + (row >> 5)] >> (row & 31)) & 1u)) continue;
        const float4 x = G[(int64_t)b * per_seq4 + i];
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
      }
    } else {
      acc = G[i];
      for (int b = 1; b < B; ++b) {
        const float4 x = G[(int64_t)b * per_seq4 + i];
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
      }
    }
    dM0[i] = acc;
  }
}

// ---- sparse gradient bookkeeping

constexpr int kTouchChunk = 16;  // steps of indices each lane holds ahead in registers

// One wavefront per memory walks the steps backwards with an N-bit "seen"
// table in LDS (N <= 2^20: 128 KiB).  Lane j owns write slot j and read
// slot j.  At step t every slot first tests its row (a row not seen at any
// later step is selected here for the last time: its bit goes into
// first[t]), then every slot marks its row; one wavefront executes its LDS
// instructions in order, so a row that is both read and written at t is
// flagged in both masks.  The final table says which rows the sequence
// selects at all.  Only wave-level ordering is needed: no workgroup
// barrier (whose fence would also wait for the mask stores and the index
// prefetch).
__global__ __launch_bounds__(kWave) void touch_kernel(const int32_t* __restrict__ widx,
                                                      const int32_t* __restrict__ ridx,
                                                      int64_t N, int64_t T, int W, int R,
                                                      uint32_t* __restrict__ seen_out,
                                                      uint64_t* __restrict__ first) {
  __shared__ uint32_t seen[kTouchMaxN / 32];
  const int64_t mem = blockIdx.x;
  const int lane = lane_id();
  const int words = (int)((N + 31) / 32);
  for (int i = lane; i < words; i += kWave) seen[i] = 0u;
  // Buffer loads and stores with out-of-range offsets instead of branches,
  // so the compiler's wait counts stay exact and the index prefetch stays
  // in flight while a chunk is walked.
  // descriptor ranges from ranges.h (touch_ok, checked on the host)
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(widx) + mem * T * W, 0, (int)ranges::table_range(T * W, 4, 0, 4),
      kBufWord3);
  const __amdgpu_buffer_rsrc_t rres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(ridx) + mem * T * R, 0, (int)ranges::table_range(T * R, 4, 0, 4),
      kBufWord3);
  const __amdgpu_buffer_rsrc_t fres = __builtin_amdgcn_make_buffer_rsrc(
      first + mem * T * 2, 0, (int)ranges::table_range(T, 16, 0, 16), kBufWord3);
  const bool ow = lane < W, orr = lane < R;
  uint32_t cw[kTouchChunk], cr[kTouchChunk], nw[kTouchChunk], nr[kTouchChunk];
  auto load = [&](uint32_t (&w)[kTouchChunk], uint32_t (&r)[kTouchChunk], int64_t c0)
      __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kTouchChunk; ++s) {
      const bool live = c0 >= 0 && c0 + s < T;
      const uint32_t wo = live && ow ? (uint32_t)((c0 + s) * W + lane) * 4u : kOffNone;
      const uint32_t ro = live && orr ? (uint32_t)((c0 + s) * R + lane) * 4u : kOffNone;
      w[s] = __builtin_amdgcn_raw_buffer_load_b32(wres, wo, 0, 0);
      r[s] = __builtin_amdgcn_raw_buffer_load_b32(rres, ro, 0, 0);
    }
  };
  // chunks from the end: a chunk covers steps [t0, t0 + kTouchChunk), clipped to [0, T)
  int64_t t0 = T > 0 ? ((T - 1) / kTouchChunk) * kTouchChunk : -1;
  load(cw, cr, t0);
  wave_sync();
  for (; t0 >= 0; t0 -= kTouchChunk) {
    load(nw, nr, t0 - kTouchChunk);  // the next chunk, in flight while this one is walked
#pragma unroll
    for (int s = kTouchChunk - 1; s >= 0; --s) {
      const int64_t t = t0 + s;
      if (t >= T) continue;  // the ragged last chunk (uniform over the wave)
      const bool vw = ow && (uint64_t)cw[s] < (uint64_t)N;
      const bool vr = orr && (uint64_t)cr[s] < (uint64_t)N;
      const uint32_t hw = vw ? cw[s] : 0u, hr = vr ? cr[s] : 0u;
      const bool fw = vw && !((seen[hw >> 5] >> (hw & 31)) & 1u);
      const bool fr = vr && !((seen[hr >> 5] >> (hr & 31)) & 1u);
      const uint64_t mw = __ballot(fw), mr = __ballot(fr);
      const u32x4 q = {(uint32_t)mw, (uint32_t)(mw >> 32), (uint32_t)mr, (uint32_t)(mr >> 32)};
      __builtin_amdgcn_raw_buffer_store_b128(q, fres, lane == 0 ? (uint32_t)t * 16u : kOffNone, 0,
                                             0);
      wave_sync();  // every test of step t before any mark
      if (vw) atomicOr(&seen[hw >> 5], 1u << (hw & 31));
      if (vr) atomicOr(&seen[hr >> 5], 1u << (hr & 31));
      wave_sync();  // the marks before step t - 1's tests
    }
#pragma unroll
    for (int s = 0; s < kTouchChunk; ++s) {
      cw[s] = nw[s];
      cr[s] = nr[s];
    }
  }
  for (int i = lane; i < words; i += kWave) seen_out[mem * words + i] = seen[i];
}

int cu_count() {
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    cu = 256;
  return cu;
}

}  // namespace

size_t scan_backward_workspace_bytes(int n_mem, int d_v, int64_t T, int W, int R) {
  const int cols = d_v < 16 ? d_v : 16;  // the narrowest tiles either mode uses
  return (size_t)n_mem * (size_t)T * (size_t)(d_v / cols) * (size_t)(W + R + 1) * sizeof(float);
}

hipError_t launch_scan_backward(int B, int H, int64_t N, int d_v, int64_t T, int W,
                                int R, const int32_t* widx, const float* wk,
                                const int32_t* ridx, const float* rw, const float* v,
                                const float* alpha, const float* beta, const float* tape,
                                const float* dout, float* G, float* dv, float* dwk, float* drw,
                                float* dalpha, float* dbeta, const uint64_t* first, float* ws,
                                hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // Tile width (measured at mid): the dense mode gathers every G row at
  // random, so whole 128-byte lines (32 columns, one wave per compute unit)
  // are fastest (14.1 ms against 17.3 with 16 columns).  In the sparse mode
  // most G gathers are dropped and the tape rows are read in order, so twice
  // the wavefronts with half the arithmetic each win (16 columns: 11.5 ms
  // against 13.4).
  const int cols = first ? (d_v < 16 ? d_v : 16) : (d_v < 32 ? d_v : 32);
  BwdArgs A{B * H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta, dout, tape, G, dv, ws,
            d_v / cols, first};
  const int groups = (A.n_mem + 7) / 8;
  const int64_t blocks = (int64_t)groups * A.ntiles * 8;
  if (cols == 32)
    hipLaunchKernelGGL((scan_bwd_kernel<32>), dim3((unsigned)blocks), dim3(kWave), 0, stream, A);
  else
    hipLaunchKernelGGL((scan_bwd_kernel<16>), dim3((unsigned)blocks), dim3(kWave), 0, stream, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = (int64_t)A.n_mem * T;
  hipLaunchKernelGGL(scan_bwd_finish, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, A,
                     dwk, drw, dalpha, dbeta);
  return hipGetLastError();
}

hipError_t launch_select_backward(const int32_t* idx, const float* w, const float* dw,
                                  int64_t units, int n, int K, float* dx1, float* dx2,
                                  hipStream_t stream) {
  if (units == 0) return hipSuccess;
  const size_t lds = (size_t)4 * 2 * (size_t)n * sizeof(float);  // <= 64 KiB for n <= 2048
  const bool wide = (n % 4) == 0 && ((uintptr_t)dx1 % 16) == 0 && ((uintptr_t)dx2 % 16) == 0;
  hipLaunchKernelGGL(select_bwd_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), lds,
                     stream, idx, w, dw, units, n, K, dx1, dx2, wide);
  return hipGetLastError();
}

hipError_t launch_state_init_backward(const float* G, int B, int H, int64_t N, int d_v,
                                      const uint32_t* seen, float* dM0, hipStream_t stream) {
  const int64_t n4 = (int64_t)H * N * d_v / 4;
  int64_t blocks = (n4 + 255) / 256;
  const int64_t cap = (int64_t)cu_count() * 8;
  if (blocks > cap) blocks = cap;
  if (seen)
    hipLaunchKernelGGL(init_bwd_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(G), reinterpret_cast<float4*>(dM0), B, n4,
                       n4, seen, N, d_v / 4);
  else
    hipLaunchKernelGGL(init_bwd_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(G), reinterpret_cast<float4*>(dM0), B, n4,
                       n4, seen, N, d_v / 4);
  return hipGetLastError();
}

hipError_t launch_touch_prepare(int B, int H, int64_t N, int64_t T, int W, int R,
                                const int32_t* widx, const int32_t* ridx, uint32_t* seen,
                                uint64_t* first, hipStream_t stream) {
  hipLaunchKernelGGL(touch_kernel, dim3((unsigned)((int64_t)B * H)), dim3(kWave), 0, stream, widx,
                     ridx, N, T, W, R, seen, first);
  return hipGetLastError();
}

}  // namespace sdm
