// Scan kernel: T sequential steps of the gated delta write and the sparse
// read (page "Riepilogo Tecnico: Sparse Delta Memory (SDM)", section
// "Meccanismo Core", items 3 and 4) for every (b,h) memory.
//
// Layout and parallelism.  The update is independent per column, so each
// memory's d_v columns are split into tiles of 128 bytes (one cache line of
// every slot row); one wavefront owns one (b,h,tile) and walks t = 0..T-1.
// Per step it gathers the W write rows and the R read rows of its tile with
// 16-byte loads (LPR lanes per row, RPI rows per instruction), applies
// Mt = alpha*M, M = Mt + (beta*k)*(v - Mt) in fp32, stores the W rows back,
// and forms o_t = sum_j r_j M_t[g_j] for its columns.  A read row that is
// also written in the same step is taken from the just-updated values (kept
// in LDS as stored, i.e. rounded to the state type) through a small LDS hash
// table keyed by row.  All memory traffic of a tile comes from one wave, so
// a later step's load of a row is ordered after the earlier step's store.
// Blocks are numbered so that all tiles of one memory land on the same XCD
// (blocks are dealt to the 8 XCDs round-robin), which shares the index,
// weight and value traffic of a memory in one L2.  Nothing here is a dense
// contraction, so there is no MFMA: the kernel is bound by HBM traffic,
// (2W + R) * tile bytes per step per tile.
#include "device_common.h"
#include "internal.h"

namespace sdm {
namespace {

constexpr int kChunk = 16;     // steps whose indices/weights/values sit in LDS at once
constexpr int kHash = 256;     // LDS hash table entries (W <= 64)

template <typename DT, int COLS>
struct Tile {
  static constexpr int ES = sizeof(DT);
  static constexpr int TB = COLS * ES;   // tile bytes (<= 128)
  static constexpr int EPL = 16 / ES;    // elements per lane per 16-byte access
  static constexpr int LPR = TB / 16;    // lanes per row
  static constexpr int RPI = kWave / LPR;  // rows per wave instruction
  static constexpr int NI = 64 / RPI;    // instructions for 64 rows
};

__device__ __forceinline__ uint32_t row_hash(int32_t row) {
  return ((uint32_t)row * 2654435761u) >> 24;
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

// Round to the state type and pack; also returns the stored values widened.
template <typename DT>
__device__ __forceinline__ uint4 pack(float (&f)[16 / sizeof(DT)]) {
  uint4 q;
  if constexpr (sizeof(DT) == 4) {
    q.x = __float_as_uint(f[0]);
    q.y = __float_as_uint(f[1]);
    q.z = __float_as_uint(f[2]);
    q.w = __float_as_uint(f[3]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = f32_to_bf16_rne(f[2 * i]);
      uint32_t hi = f32_to_bf16_rne(f[2 * i + 1]);
      w[i] = lo | (hi << 16);
      f[2 * i] = __uint_as_float(lo << 16);
      f[2 * i + 1] = __uint_as_float(hi << 16);
    }
    q = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return q;
}

template <typename DT, int COLS>
__global__ __launch_bounds__(kWave) void scan_kernel(
    DT* __restrict__ M, int n_mem, int64_t N, int d_v, int64_t T, int W, int R,
    const int32_t* __restrict__ widx, const float* __restrict__ wk,
    const int32_t* __restrict__ ridx, const float* __restrict__ rw, const float* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ out,
    int ntiles) {
  using TL = Tile<DT, COLS>;
  constexpr int EPL = TL::EPL, LPR = TL::LPR, RPI = TL::RPI, NI = TL::NI;

  __shared__ int32_t s_widx[kChunk * 64];
  __shared__ float s_wk[kChunk * 64];
  __shared__ int32_t s_ridx[kChunk * 64];
  __shared__ float s_rw[kChunk * 64];
  __shared__ float s_v[kChunk * COLS];
  __shared__ float s_a[kChunk], s_b[kChunk];
  __shared__ int32_t s_hash[kHash];
  __shared__ int32_t s_fwd[64];
  __shared__ uint4 s_upd[64 * LPR];

  // XCD-aware numbering: bid = ((g * ntiles) + tile) * 8 + x, memory = g*8 + x.
  const int bid = blockIdx.x;
  const int x = bid & 7;
  const int rest = bid >> 3;
  const int tile = rest % ntiles;
  const int mem = (rest / ntiles) * 8 + x;
  if (mem >= n_mem) return;

  const int lane = lane_id();
  const int lr = lane / LPR;  // row slot inside one instruction
  const int lc = lane % LPR;  // 16-byte column chunk inside the tile
  const int64_t col0 = (int64_t)tile * COLS + lc * EPL;
  DT* const Mm = M + (int64_t)mem * N * d_v;
  const uint32_t Nu = (uint32_t)N;

  for (int h = lane; h < kHash; h += kWave) s_hash[h] = 0;

  for (int64_t t0 = 0; t0 < T; t0 += kChunk) {
    const int steps = (int)((T - t0) < kChunk ? (T - t0) : kChunk);
    wave_sync();
    {  // stage this chunk's per-step inputs in LDS
      const int64_t base = (int64_t)mem * T + t0;
      for (int e = lane; e < steps * W; e += kWave) {
        s_widx[e] = widx[base * W + e];
        s_wk[e] = wk[base * W + e];
      }
      for (int e = lane; e < steps * R; e += kWave) {
        s_ridx[e] = ridx[base * R + e];
        s_rw[e] = rw[base * R + e];
      }
      for (int e = lane; e < steps * COLS; e += kWave) {
        const int s = e / COLS, c = e % COLS;
        s_v[e] = v[(base + s) * d_v + (int64_t)tile * COLS + c];
      }
      for (int e = lane; e < steps; e += kWave) {
        s_a[e] = alpha[base + e];
        s_b[e] = beta[base + e];
      }
    }
    wave_sync();

    for (int s = 0; s < steps; ++s) {
      const int32_t* sw = s_widx + s * W;
      const int32_t* sr = s_ridx + s * R;
      // gathers: write rows, then read rows
      uint4 wv[NI], rv[NI];
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int j = k * RPI + lr;
        wv[k] = make_uint4(0, 0, 0, 0);
        if (j < W) {
          const int32_t row = sw[j];
          if ((uint32_t)row < Nu)
            wv[k] = *reinterpret_cast<const uint4*>(Mm + (int64_t)row * d_v + col0);
        }
      }
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int j = k * RPI + lr;
        rv[k] = make_uint4(0, 0, 0, 0);
        if (j < R) {
          const int32_t row = sr[j];
          if ((uint32_t)row < Nu)
            rv[k] = *reinterpret_cast<const uint4*>(Mm + (int64_t)row * d_v + col0);
        }
      }
      // same-step read-after-write: hash the write rows, look up read rows
      int my_slot = -1;
      if (lane < W) {
        const int32_t row = sw[lane];
        if ((uint32_t)row < Nu) {
          uint32_t hh = row_hash(row);
          while (atomicCAS(&s_hash[hh], 0, lane + 1) != 0) hh = (hh + 1) & (kHash - 1);
          my_slot = (int)hh;
        }
      }
      wave_sync();
      if (lane < R) {
        const int32_t row = sr[lane];
        int fwd = -1;
        uint32_t hh = row_hash(row);
        for (;;) {
          const int e = s_hash[hh];
          if (e == 0) break;
          if (sw[e - 1] == row) {
            fwd = e - 1;
            break;
          }
          hh = (hh + 1) & (kHash - 1);
        }
        s_fwd[lane] = fwd;
      }
      // gated delta write
      const float a = s_a[s], b = s_b[s];
      float vv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) vv[e] = s_v[s * COLS + lc * EPL + e];
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int j = k * RPI + lr;
        if (j < W) {
          const int32_t row = sw[j];
          if ((uint32_t)row < Nu) {
            const float g = b * s_wk[s * W + j];
            float m[EPL];
            unpack<DT>(wv[k], m);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const float mt = a * m[e];
              m[e] = fmaf(g, vv[e] - mt, mt);
            }
            const uint4 q = pack<DT>(m);
            *reinterpret_cast<uint4*>(Mm + (int64_t)row * d_v + col0) = q;
            s_upd[j * LPR + lc] = q;
          }
        }
      }
      wave_sync();
      // sparse read of the rows as stored after the write
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int j = k * RPI + lr;
        if (j < R) {
          const int f = s_fwd[j];
          const uint4 q = f >= 0 ? s_upd[f * LPR + lc] : rv[k];
          const float r = s_rw[s * R + j];
          float m[EPL];
          unpack<DT>(q, m);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fmaf(r, m[e], acc[e]);
        }
      }
#pragma unroll
      for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], o);
      }
      if (lr == 0) {
        float* o = out + ((int64_t)mem * T + t0 + s) * d_v + col0;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<float4*>(o + e) = make_float4(acc[e], acc[e + 1], acc[e + 2],
                                                          acc[e + 3]);
      }
      wave_sync();
      if (my_slot >= 0) s_hash[my_slot] = 0;
    }
  }
}

template <typename DT, int COLS>
hipError_t launch(void* M, int n_mem, int64_t N, int d_v, int64_t T, int W, int R,
                  const int32_t* widx, const float* wk, const int32_t* ridx, const float* rw,
                  const float* v, const float* alpha, const float* beta, float* out,
                  hipStream_t stream) {
  const int ntiles = d_v / COLS;
  const int groups = (n_mem + 7) / 8;
  const int64_t blocks = (int64_t)groups * ntiles * 8;
  hipLaunchKernelGGL((scan_kernel<DT, COLS>), dim3((unsigned)blocks), dim3(kWave), 0, stream,
                     reinterpret_cast<DT*>(M), n_mem, N, d_v, T, W, R, widx, wk, ridx, rw, v,
                     alpha, beta, out, ntiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(void* M, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W,
                       int R, const int32_t* widx, const float* wk, const int32_t* ridx,
                       const float* rw, const float* v, const float* alpha, const float* beta,
                       float* out, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int n_mem = B * H;
  if (dtype == 0) {
    if (d_v == 16)
      return launch<float, 16>(M, n_mem, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta,
                               out, stream);
    return launch<float, 32>(M, n_mem, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta, out,
                             stream);
  }
  if (d_v == 16)
    return launch<uint16_t, 16>(M, n_mem, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta,
                                out, stream);
  if (d_v == 32)
    return launch<uint16_t, 32>(M, n_mem, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta,
                                out, stream);
  return launch<uint16_t, 64>(M, n_mem, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta,
                              out, stream);
}

}  // namespace sdm
