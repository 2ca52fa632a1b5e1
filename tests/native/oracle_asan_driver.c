/* Drives the CPU oracle through selection, the scan (fp32, bf16 and fp8 E4M3
 * state) and the backward on small random inputs, so that the oracle can be
 * built and run under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Exits non-zero on any oracle error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_select(const float*, const float*, int64_t, int, int, int32_t*, float*, double*);
int oracle_state_init(void*, int, const float*, int, int, int64_t, int);
int oracle_scan(void*, int, int64_t, int, int64_t, int, int, const int32_t*, const double*,
                const int32_t*, const double*, const float*, const float*, const float*, float*,
                int, int);
int oracle_step_decode(void*, int, int, int, int, int, int, int, const float*, const float*,
                       const float*, const float*, const float*, const float*, const float*,
                       float*, int32_t*, int32_t*);
int oracle_scan_backward(const float*, int64_t, int, int64_t, int, int, const int32_t*,
                         const double*, const int32_t*, const double*, const float*, const float*,
                         const float*, const float*, double*, double*, double*, double*, double*,
                         double*, float*, float*, float*);
int oracle_select_backward(const int32_t*, const double*, const double*, int64_t, int, int,
                           double*, double*);
const char* oracle_last_error(void);

static uint64_t s = 0x9E3779B97F4A7C15ull;
static float urand(void) { /* xorshift64*, uniform in [-1, 1) */
  s ^= s >> 12; s ^= s << 25; s ^= s >> 27;
  return (float)((s * 2685821657736338717ull) >> 40) / (float)(1 << 23) - 1.0f;
}

#define CHECK(x) do { if ((x) != 0) { fprintf(stderr, "%s: %s\n", #x, oracle_last_error()); return 1; } } while (0)

int main(void) {
  enum { n = 16, N = n * n, D = 32, T = 40, W = 7, R = 5, B = 2, H = 1 };
  float *s1 = malloc(sizeof(float) * T * n), *s2 = malloc(sizeof(float) * T * n);
  float *q1 = malloc(sizeof(float) * T * n), *q2 = malloc(sizeof(float) * T * n);
  float *v = malloc(sizeof(float) * T * D), *al = malloc(sizeof(float) * T), *be = malloc(sizeof(float) * T);
  float *M0 = malloc(sizeof(float) * N * D), *dout = malloc(sizeof(float) * T * D);
  for (int i = 0; i < T * n; ++i) { s1[i] = urand(); s2[i] = urand(); q1[i] = urand(); q2[i] = urand(); }
  for (int i = 0; i < T * D; ++i) { v[i] = urand(); dout[i] = urand(); }
  for (int i = 0; i < T; ++i) { al[i] = 0.95f + 0.05f * urand(); be[i] = 0.5f + 0.5f * urand(); }
  for (int i = 0; i < N * D; ++i) M0[i] = 0.02f * urand();
  int32_t *wi = malloc(sizeof(int32_t) * T * W), *ri = malloc(sizeof(int32_t) * T * R);
  double *wk = malloc(sizeof(double) * T * W), *rw = malloc(sizeof(double) * T * R);
  float *ws = malloc(sizeof(float) * T * W);
  CHECK(oracle_select(s1, s2, T, n, W, wi, ws, wk));
  CHECK(oracle_select(q1, q2, T, n, R, ri, NULL, rw));
  for (int dt = 0; dt < 3; ++dt) {
    size_t es = dt == 0 ? 4 : (dt == 1 ? 2 : 1);
    void* M = malloc(es * (size_t)B * H * N * D);
    float* out = malloc(sizeof(float) * T * D);
    CHECK(oracle_state_init(M, dt, M0, B, H, N, D));
    CHECK(oracle_scan(M, dt, N, D, T, W, R, wi, wk, ri, rw, v, al, be, out, 0, D));
    CHECK(oracle_scan(M, dt, N, D, T, W, R, wi, wk, ri, rw, v, al, be, out, 3, 17));
    if (dt < 2) {
      float* o2 = malloc(sizeof(float) * B * D);
      int32_t *w2 = malloc(sizeof(int32_t) * B * W), *r2 = malloc(sizeof(int32_t) * B * R);
      float *s1b = malloc(sizeof(float) * B * n), *s2b = malloc(sizeof(float) * B * n);
      float *q1b = malloc(sizeof(float) * B * n), *q2b = malloc(sizeof(float) * B * n);
      memcpy(s1b, s1, sizeof(float) * B * n); memcpy(s2b, s2, sizeof(float) * B * n);
      memcpy(q1b, q1, sizeof(float) * B * n); memcpy(q2b, q2, sizeof(float) * B * n);
      CHECK(oracle_step_decode(M, dt, B, H, n, D, W, R, s1b, s2b, q1b, q2b, v, al, be, o2, w2, r2));
      free(o2); free(w2); free(r2); free(s1b); free(s2b); free(q1b); free(q2b);
    }
    free(M); free(out);
  }
  double *G = calloc((size_t)N * D, sizeof(double)), *dv = malloc(sizeof(double) * T * D);
  double *dwk = malloc(sizeof(double) * T * W), *drw = malloc(sizeof(double) * T * R);
  double *da = malloc(sizeof(double) * T), *db = malloc(sizeof(double) * T);
  float *tape = malloc(sizeof(float) * T * W * D), *MT = malloc(sizeof(float) * N * D);
  float *rtape = malloc(sizeof(float) * T * R * D);
  CHECK(oracle_scan_backward(M0, N, D, T, W, R, wi, wk, ri, rw, v, al, be, dout, G, dv, dwk, drw,
                             da, db, tape, rtape, MT));
  double *dx1 = malloc(sizeof(double) * T * n), *dx2 = malloc(sizeof(double) * T * n);
  CHECK(oracle_select_backward(wi, wk, dwk, T, n, W, dx1, dx2));
  /* a rejected call must fail cleanly */
  wi[3] = wi[4];
  if (oracle_scan_backward(M0, N, D, T, W, R, wi, wk, ri, rw, v, al, be, dout, G, dv, dwk, drw, da,
                           db, NULL, NULL, NULL) == 0) return 2;
  free(s1); free(s2); free(q1); free(q2); free(v); free(al); free(be); free(M0); free(dout);
  free(wi); free(ri); free(wk); free(rw); free(ws); free(G); free(dv); free(dwk); free(drw);
  free(da); free(db); free(tape); free(rtape); free(MT); free(dx1); free(dx2);
  puts("ok");
  return 0;
}
