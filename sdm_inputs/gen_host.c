/* Seeded synthetic-input generator, host side (plain C, built with gcc
 * -ffp-contract=off so every float operation below is one IEEE binary32
 * operation with round-to-nearest-even, in the order written).
 *
 * This module holds none of the SDM method's arithmetic: it only produces the
 * random inputs (sub-scores, values, gates, initial memory) that both the
 * CPU oracle and the GPU path consume.  A device twin in gen_device.hip
 * implements the same definition; the two agree bit for bit because every
 * step is either integer arithmetic or a single correctly rounded float op.
 *
 * Definition
 *   bits:    Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 *            numbers: as easy as 1, 2, 3", SC'11): counter (c0..c3), key
 *            (k0,k1); each round multiplies c0 and c2 by 0xD2511F53 and
 *            0xCD9E8D57 into hi/lo halves and permutes
 *            (hi1^c1^k0, lo1, hi0^c3^k1, lo0); the key is bumped by the Weyl
 *            constants 0x9E3779B9 / 0xBB67AE85 between rounds.
 *   element: value number e (uint64) of a stream (seed, tag) uses Philox call
 *            counter = (lo32(e>>2), hi32(e>>2), 0, 0), key = (seed, tag), and
 *            word e&3 of the result.
 *   uniform: u = (w >> 8) * 2^-24 in [0,1).
 *   normal:  Box-Muller on word pairs (w0,w1) and (w2,w3):
 *            u1 = ((wa>>8)+1)*2^-24 in (0,1], u2 = (wb>>8)*2^-24,
 *            r = sqrt(-2 ln u1), z_a = r cos(2 pi u2), z_b = r sin(2 pi u2),
 *            with ln, sin and cos evaluated by the fixed polynomials below
 *            (not libm), then z + 0.0f so that -0.0 never occurs.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void sdm_gen_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)x0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)x2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t y0 = hi1 ^ x1 ^ k0;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    x0 = y0;
    x1 = lo1;
    x2 = y2;
    x3 = lo0;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

static float f_from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}
static uint32_t bits_from_f(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* Natural log of x in [2^-24, 1]: x = f * 2^e with f in [sqrt(1/2), sqrt(2)),
 * ln f = 2 atanh(s), s = (f-1)/(f+1), odd series to s^11. */
static float gen_ln(float x) {
  uint32_t b = bits_from_f(x);
  int e = (int)((b >> 23) & 0xFFu) - 127;
  uint32_t mb = (b & 0x007FFFFFu) | 0x3F800000u;
  float f = f_from_bits(mb);
  if (f > 1.41421353816986083984375f) {
    mb -= 0x00800000u;
    f = f_from_bits(mb);
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

/* cos and sin of 2*pi*j/2^24 for a 24-bit integer j: exact quadrant split,
 * phi = (j mod 2^22) * 2^-22 * pi/2 in [0, pi/2), then
 *   sin phi = phi (1 - p/3! + p^2/5! - ... + p^6/13!),
 *   cos phi = 1 - p/2! + p^2/4! - ... - p^7/14!,   p = phi^2,
 * by Horner's rule. */
static void gen_sincos_turn(uint32_t j, float* c_out, float* s_out) {
  uint32_t q = j >> 22;
  float y = (float)(j & 0x3FFFFFu) * 2.384185791015625e-07f; /* 2^-22 */
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
  float c, s;
  switch (q) {
    case 0: c = cp; s = sn; break;
    case 1: c = -sn; s = cp; break;
    case 2: c = -cp; s = -sn; break;
    default: c = sn; s = -cp; break;
  }
  *c_out = c;
  *s_out = s;
}

static void gen_box_muller(uint32_t wa, uint32_t wb, float* za, float* zb) {
  float u1 = (float)((wa >> 8) + 1u) * 5.9604644775390625e-08f; /* 2^-24 */
  float l = gen_ln(u1);
  float r = sqrtf(-2.0f * l);
  float c, s;
  gen_sincos_turn(wb >> 8, &c, &s);
  *za = r * c + 0.0f;
  *zb = r * s + 0.0f;
}

/* Kinds of stream. */
enum { GEN_NORMAL = 0, GEN_UNIFORM = 1 };

/* The four values of Philox call number `call` of stream (seed, tag). */
static void gen_quad(uint32_t seed, uint32_t tag, uint64_t call, int kind, float out[4]) {
  uint32_t ctr[4] = {(uint32_t)call, (uint32_t)(call >> 32), 0u, 0u};
  uint32_t key[2] = {seed, tag};
  uint32_t w[4];
  sdm_gen_philox4x32_10(ctr, key, w);
  if (kind == GEN_UNIFORM) {
    for (int k = 0; k < 4; ++k) out[k] = (float)(w[k] >> 8) * 5.9604644775390625e-08f;
  } else {
    gen_box_muller(w[0], w[1], &out[0], &out[1]);
    gen_box_muller(w[2], w[3], &out[2], &out[3]);
  }
}

/* Sequential reader of one stream: recomputes a Philox call only when the
 * requested value number leaves the current group of four. */
typedef struct {
  uint32_t seed, tag;
  int kind;
  uint64_t call;
  int valid;
  float q[4];
} gen_stream;

static float gen_stream_get(gen_stream* st, uint64_t e) {
  uint64_t call = e >> 2;
  if (!st->valid || call != st->call) {
    gen_quad(st->seed, st->tag, call, st->kind, st->q);
    st->call = call;
    st->valid = 1;
  }
  return st->q[e & 3u];
}

/* Value number e of stream (seed, tag). */
float sdm_gen_value(uint32_t seed, uint32_t tag, uint64_t e, int kind) {
  float q[4];
  gen_quad(seed, tag, e >> 2, kind, q);
  return q[e & 3u];
}

/* Fill a 4-D block dst[nb][nh][nt][len] of a logical tensor [B][H][T][len].
 * Element (b,h,t,i) with b=b0+bb, h=h0+hh, t=t0+tt has flat number
 *   e = ((b*H + h)*T + t)*len + i.
 * kind GEN_NORMAL:  value = scale * z(seed, tag, e)            (one rounding)
 *                   or, with mix_tag >= 0,
 *                   value = z(seed, mix_tag, (b*T + t)*len + i) + mixw * z(seed, tag, e)
 * kind GEN_UNIFORM: value = lo + (hi - lo) * u(seed, tag, e)
 * All arithmetic is binary32 in the order written. */
void sdm_gen_fill_block(float* dst, int64_t nb, int64_t nh, int64_t nt, int64_t len,
                        int64_t B, int64_t H, int64_t T, int64_t b0, int64_t h0, int64_t t0,
                        uint32_t seed, uint32_t tag, int kind, float scale, float lo, float hi,
                        int mix_tag, float mixw) {
  (void)B;
  float width = hi - lo;
  gen_stream own = {seed, tag, kind, 0, 0, {0, 0, 0, 0}};
  gen_stream mix = {seed, (uint32_t)(mix_tag < 0 ? 0 : mix_tag), GEN_NORMAL, 0, 0, {0, 0, 0, 0}};
  for (int64_t bb = 0; bb < nb; ++bb)
    for (int64_t hh = 0; hh < nh; ++hh)
      for (int64_t tt = 0; tt < nt; ++tt) {
        int64_t b = b0 + bb, h = h0 + hh, t = t0 + tt;
        float* row = dst + ((bb * nh + hh) * nt + tt) * len;
        uint64_t ebase = (uint64_t)(((b * H + h) * T + t) * len);
        uint64_t mbase = (uint64_t)((b * T + t) * len);
        for (int64_t i = 0; i < len; ++i) {
          float val;
          if (kind == GEN_UNIFORM) {
            float u = gen_stream_get(&own, ebase + (uint64_t)i);
            val = lo + width * u;
          } else if (mix_tag >= 0) {
            float g = gen_stream_get(&mix, mbase + (uint64_t)i);
            float z = gen_stream_get(&own, ebase + (uint64_t)i);
            val = g + mixw * z;
          } else {
            val = scale * gen_stream_get(&own, ebase + (uint64_t)i);
          }
          row[i] = val;
        }
      }
}
