// Seeded synthetic-input generator, device side (HIP for gfx950).
//
// Same definition as gen_host.c (Philox4x32-10 bits, uniform and Box-Muller
// normal transforms with fixed polynomials), written separately for the GPU.
// Built with -ffp-contract=off: every float operation is one binary32
// operation with round-to-nearest-even, in the order written, and division
// and sqrt are the correctly rounded forms (HIP's default for fp32), so a
// value here equals the host value bit for bit.  This file is input
// generation only; it contains none of the SDM method's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;

__device__ inline void philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                              uint32_t k1, uint32_t out[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kW0;
      k1 += kW1;
    }
    uint32_t lo0 = kM0 * c0, hi0 = __umulhi(kM0, c0);
    uint32_t lo1 = kM1 * c2, hi1 = __umulhi(kM1, c2);
    uint32_t y0 = hi1 ^ c1 ^ k0;
    uint32_t y2 = hi0 ^ c3 ^ k1;
    c0 = y0;
    c1 = lo1;
    c2 = y2;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

__device__ inline float ln_unit(float x) {
  uint32_t b = __float_as_uint(x);
  int e = (int)((b >> 23) & 0xFFu) - 127;
  uint32_t mb = (b & 0x007FFFFFu) | 0x3F800000u;
  float f = __uint_as_float(mb);
  if (f > 1.41421353816986083984375f) {
    mb -= 0x00800000u;
    f = __uint_as_float(mb);
    e += 1;
  }
  float s = (f - 1.0f) / (f + 1.0f);
  float z = s * s;
  float p = 0.181818181818181818f;
  p = p * z + 0.222222222222222222f;
  p = p * z + 0.285714285714285714f;
  p = p * z + 0.4f;
  p = p * z + 0.666666666666666667f;
  p = p * z + 2.0f;
  float lnf = s * p;
  float ef = (float)e;
  return ef * 0.693145751953125f + (ef * 1.42860682030941723212e-06f + lnf);
}

__device__ inline void sincos_turn(uint32_t j, float& c, float& s) {
  uint32_t q = j >> 22;
  float y = (float)(j & 0x3FFFFFu) * 2.384185791015625e-07f;
  float phi = y * 1.57079632679489661923f;
  float p = phi * phi;
  float sp = 1.60590438368216145994e-10f;
  sp = sp * p - 2.50521083854417187751e-08f;
  sp = sp * p + 2.75573192239858906526e-06f;
  sp = sp * p - 1.98412698412698412698e-04f;
  sp = sp * p + 8.33333333333333333333e-03f;
  sp = sp * p - 1.66666666666666666667e-01f;
  sp = sp * p + 1.0f;
  float sn = phi * sp;
  float cp = -1.14707455977297247139e-11f;
  cp = cp * p + 2.08767569878680989792e-09f;
  cp = cp * p - 2.75573192239858906526e-07f;
  cp = cp * p + 2.48015873015873015873e-05f;
  cp = cp * p - 1.38888888888888888889e-03f;
  cp = cp * p + 4.16666666666666666667e-02f;
  cp = cp * p - 0.5f;
  cp = cp * p + 1.0f;
  switch (q) {
    case 0: c = cp; s = sn; break;
    case 1: c = -sn; s = cp; break;
    case 2: c = -cp; s = -sn; break;
    default: c = sn; s = -cp; break;
  }
}

// Value number e of stream (seed, tag): kind 0 normal, 1 uniform.
__device__ inline float value_at(uint32_t seed, uint32_t tag, uint64_t e, int kind) {
  uint64_t call = e >> 2;
  uint32_t w[4];
  philox((uint32_t)call, (uint32_t)(call >> 32), 0u, 0u, seed, tag, w);
  unsigned pos = (unsigned)(e & 3u);
  if (kind == 1) return (float)(w[pos] >> 8) * 5.9604644775390625e-08f;
  uint32_t wa = pos < 2 ? w[0] : w[2];
  uint32_t wb = pos < 2 ? w[1] : w[3];
  float u1 = (float)((wa >> 8) + 1u) * 5.9604644775390625e-08f;
  float l = ln_unit(u1);
  float r = __builtin_sqrtf(-2.0f * l);
  float c, s;
  sincos_turn(wb >> 8, c, s);
  float z = (pos & 1u) ? r * s : r * c;
  return z + 0.0f;
}

__global__ void fill_block_kernel(float* __restrict__ dst, int64_t total, int64_t nh, int64_t nt,
                                  int64_t len, int64_t H, int64_t T, int64_t b0, int64_t h0,
                                  int64_t t0, uint32_t seed, uint32_t tag, int kind, float scale,
                                  float lo, float width, int mix_tag, float mixw) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total; k += stride) {
    int64_t i = k % len;
    int64_t r = k / len;
    int64_t tt = r % nt;
    r /= nt;
    int64_t hh = r % nh;
    int64_t bb = r / nh;
    int64_t b = b0 + bb, h = h0 + hh, t = t0 + tt;
    uint64_t e = (uint64_t)(((b * H + h) * T + t) * len + i);
    float val;
    if (kind == 1) {
      val = lo + width * value_at(seed, tag, e, 1);
    } else if (mix_tag >= 0) {
      uint64_t em = (uint64_t)((b * T + t) * len + i);
      float g = value_at(seed, (uint32_t)mix_tag, em, 0);
      float z = value_at(seed, tag, e, 0);
      val = g + mixw * z;
    } else {
      val = scale * value_at(seed, tag, e, 0);
    }
    dst[k] = val;
  }
}

}  // namespace

// Device fill of dst[nb][nh][nt][len] (device pointer, contiguous) with the
// same values sdm_gen_fill_block produces on the host.  Enqueued on `stream`
// (a hipStream_t); returns the hipError_t of the launch (0 on success).
extern "C" int sdm_gen_fill_block_device(float* dst, int64_t nb, int64_t nh, int64_t nt,
                                         int64_t len, int64_t B, int64_t H, int64_t T, int64_t b0,
                                         int64_t h0, int64_t t0, uint32_t seed, uint32_t tag,
                                         int kind, float scale, float lo, float hi, int mix_tag,
                                         float mixw, void* stream) {
  (void)B;
  int64_t total = nb * nh * nt * len;
  if (total <= 0) return 0;
  int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  float width = hi - lo;
  hipLaunchKernelGGL(fill_block_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                     (hipStream_t)stream, dst, total, nh, nt, len, H, T, b0, h0, t0, seed, tag,
                     kind, scale, lo, width, mix_tag, mixw);
  return (int)hipGetLastError();
}
