/* CPU oracle for the Sparse Delta Memory (SDM) recurrent step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check
 * and the benchmark's CPU-baseline leg may load this library.  The GPU
 * product path never calls, links or falls back to it, and it shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes.  Source pages: "Riepilogo Tecnico: Sparse Delta Memory
 * (SDM)" (gist.science/it/paper/2607.07386), sections "Meccanismo Core",
 * items 1-4, and "Stato Iniziale Appreso"; the same content appears in
 * "技術要約：Sparse Delta Memory (SDM)" (gist.science/ja/paper/2607.07386),
 * sections "コアメカニズム" and "学習された初期状態".
 *
 *  - Memory: an explicit table M with N = n*n rows of d_v values (item 1).
 *  - Selection (item 2): the key (or query) is split in two halves x1, x2 of
 *    length n; slot f = a*n + b scores x1[a] + x2[b].  The top-K slots are
 *    found without forming all N scores, through
 *    topk(x1 (+) x2) = topk(topk(x1) (+) topk(x2)):
 *      stage 1: the K best indices of each half, in the order
 *               "larger value first, lower index first on equal values";
 *      stage 2: the K best of the K*K candidate sums
 *               sigma = fl32(x1[a] + x2[b]) in the order
 *               "larger sigma first, lower flat index f first on equal sigma".
 *    K = W for the write selection (from s1, s2) and K = R for the read
 *    selection (from q1, q2).
 *  - Selection weights: softmax over the K selected sigma (the pages name the
 *    weights k_t^(i) but do not say how they are formed; softmax over the
 *    selected scores is the reading used throughout).  Computed in double.
 *  - Gated delta write on the W selected rows (item 3):
 *      Mt[i] = alpha_t * M[i];  M[i] = Mt[i] + beta_t * k_i * (v_t - Mt[i]);
 *    every other row is left as it is.  Computed in double from the stored
 *    value and rounded once to the state type (fp32, or bf16 with
 *    round-to-nearest-even).
 *  - Sparse read (item 4): o_t = sum_j r_j * M[g_j] over the R selected read
 *    rows, taken from the stored memory after this step's write.
 *    Accumulated in double, rounded once to fp32.
 *  - Learned initial state: every sequence's memory starts as a copy of M0
 *    (fp32; rounded to bf16 with round-to-nearest-even for bf16 state, to
 *    fp8 E4M3 likewise for fp8 state).
 *  - fp8 E4M3 state: the stored code is decided by the binary32 update, so
 *    for that state type the write is taken in binary32 in a fixed order
 *    (see oracle_scan) and then rounded to E4M3.
 *
 * All inputs must be finite; the functions return a non-zero status and set
 * a message otherwise.  Plain, slow and single-threaded on purpose.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static __thread char g_msg[256];

const char* oracle_last_error(void) { return g_msg; }

static int fail(const char* what) {
  snprintf(g_msg, sizeof g_msg, "%s", what);
  return 1;
}

/* ------------------------------------------------------------------ bf16 */

static double bf16_to_double(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 value (ties to even) and return its bits.
 * bf16 keeps 8 significant bits and the binary32 exponent range, so the grid
 * spacing near |x| in [2^(e-1), 2^e) is 2^(e-8), and never finer than the
 * subnormal spacing 2^-133. */
static uint16_t bf16_from_double(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000u : 0x0000u;
  int e;
  (void)frexp(x, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  double r = nearbyint(ldexp(x, -q));
  double y = ldexp(r, q);
  float f = (float)y;
  uint32_t b;
  memcpy(&b, &f, 4);
  return (uint16_t)(b >> 16);
}

/* ------------------------------------------------------------------ fp8
 * OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; no infinities; codes 0x7F and 0xFF are NaN; largest finite
 * value 448 = 1.75 * 2^8; normal values from 2^-6, subnormals m * 2^-9 for
 * m = 1..7.  Encoding rounds to the nearest representable value, ties to the
 * even code, and clamps magnitudes beyond 448 to 448 (a finite state never
 * needs more: every write is a convex combination of alpha*M and v). */

static double fp8_to_double(uint8_t c) {
  int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return sgn ? -mag : mag;
}

static uint8_t fp8_from_float(float x) {
  uint8_t sgn = signbit(x) ? 0x80u : 0x00u;
  double a = fabs((double)x);
  if (a == 0.0) return sgn;
  int e;
  (void)frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int q = e - 4;      /* spacing of 3-mantissa-bit values in that binade */
  if (q < -9) q = -9; /* subnormal spacing */
  double r = ldexp(nearbyint(ldexp(a, -q)), q); /* exact scaling; rint is ties-to-even */
  if (r > 448.0) r = 448.0;
  if (r < ldexp(1.0, -6)) return (uint8_t)(sgn | (uint8_t)ldexp(r, 9));
  int er;
  double fr = frexp(r, &er); /* r = fr * 2^er, fr in [0.5, 1) */
  int E = er - 1 + 7;
  int M = (int)ldexp(fr * 2.0 - 1.0, 3);
  return (uint8_t)(sgn | (uint8_t)(E << 3) | (uint8_t)M);
}

/* ------------------------------------------------------------- selection */

/* Half order: index i goes before index j. */
static int half_before(const float* x, int i, int j) {
  return x[i] > x[j] || (x[i] == x[j] && i < j);
}

/* The first K indices of x[0..n) in half order, written to best[0..K) in
 * that order.  Kept as a sorted buffer of the best K seen so far. */
static void topk_half(const float* x, int n, int K, int* best) {
  int cnt = 0;
  for (int i = 0; i < n; ++i) {
    if (cnt == K && !half_before(x, i, best[K - 1])) continue;
    int pos = cnt < K ? cnt : K - 1;
    while (pos > 0 && half_before(x, i, best[pos - 1])) {
      best[pos] = best[pos - 1];
      --pos;
    }
    best[pos] = i;
    if (cnt < K) ++cnt;
  }
}

/* Candidate order: (sigma, f) goes before (sigma2, f2). */
static int cand_before(float s, int32_t f, float s2, int32_t f2) {
  return s > s2 || (s == s2 && f < f2);
}

static int all_finite(const float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

/* One selection: K slots of the product-key table spanned by halves x1, x2. */
static void select_one(const float* x1, const float* x2, int n, int K, int* A, int* Bv,
                       float* cs, int32_t* cf, int32_t* idx, float* score, double* weight) {
  topk_half(x1, n, K, A);
  topk_half(x2, n, K, Bv);
  int cnt = 0;
  for (int ia = 0; ia < K; ++ia) {
    for (int ib = 0; ib < K; ++ib) {
      int a = A[ia], b = Bv[ib];
      float s = x1[a] + x2[b]; /* one binary32 addition, round to nearest even */
      int32_t f = (int32_t)a * (int32_t)n + (int32_t)b;
      if (cnt == K && !cand_before(s, f, cs[K - 1], cf[K - 1])) continue;
      int pos = cnt < K ? cnt : K - 1;
      while (pos > 0 && cand_before(s, f, cs[pos - 1], cf[pos - 1])) {
        cs[pos] = cs[pos - 1];
        cf[pos] = cf[pos - 1];
        --pos;
      }
      cs[pos] = s;
      cf[pos] = f;
      if (cnt < K) ++cnt;
    }
  }
  double top = (double)cs[0];
  double z = 0.0;
  for (int j = 0; j < K; ++j) z += exp((double)cs[j] - top);
  for (int j = 0; j < K; ++j) {
    idx[j] = cf[j];
    if (score) score[j] = cs[j];
    weight[j] = exp((double)cs[j] - top) / z;
  }
}

/* units independent selections: x1, x2 [units, n]; idx, score, weight
 * [units, K] in the selection order.  score may be NULL. */
int oracle_select(const float* x1, const float* x2, int64_t units, int n, int K, int32_t* idx,
                  float* score, double* weight) {
  if (!x1 || !x2 || !idx || !weight) return fail("null pointer");
  if (units < 0 || n < 1 || K < 1 || K > n) return fail("bad sizes");
  if ((int64_t)n * n >= ((int64_t)1 << 31)) return fail("n*n must fit int32 flat indices");
  int* A = (int*)malloc(sizeof(int) * (size_t)K);
  int* Bv = (int*)malloc(sizeof(int) * (size_t)K);
  float* cs = (float*)malloc(sizeof(float) * (size_t)K);
  int32_t* cf = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
  if (!A || !Bv || !cs || !cf) {
    free(A); free(Bv); free(cs); free(cf);
    return fail("out of memory");
  }
  int rc = 0;
  for (int64_t u = 0; u < units; ++u) {
    const float* a = x1 + u * n;
    const float* b = x2 + u * n;
    if (!all_finite(a, n) || !all_finite(b, n)) {
      rc = fail("non-finite sub-score");
      break;
    }
    select_one(a, b, n, K, A, Bv, cs, cf, idx + u * K, score ? score + u * K : NULL,
               weight + u * K);
  }
  free(A); free(Bv); free(cs); free(cf);
  return rc;
}

/* ----------------------------------------------------------------- state */

/* M[b,h] = M0[h] for all b.  dtype 0: fp32 copy; 1: bf16, nearest even;
 * 2: fp8 E4M3, nearest even.  M [B,H,N,d_v] (float, uint16 or uint8),
 * M0 [H,N,d_v] float. */
int oracle_state_init(void* M, int dtype, const float* M0, int B, int H, int64_t N, int d_v) {
  if (!M || !M0) return fail("null pointer");
  if (B < 1 || H < 1 || N < 1 || d_v < 1 || dtype < 0 || dtype > 2) return fail("bad sizes");
  int64_t per = N * d_v;
  if (!all_finite(M0, per * H)) return fail("non-finite M0");
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const float* src = M0 + (int64_t)h * per;
      int64_t off = ((int64_t)b * H + h) * per;
      if (dtype == 0) {
        memcpy((float*)M + off, src, sizeof(float) * (size_t)per);
      } else if (dtype == 1) {
        uint16_t* dst = (uint16_t*)M + off;
        for (int64_t i = 0; i < per; ++i) dst[i] = bf16_from_double((double)src[i]);
      } else {
        uint8_t* dst = (uint8_t*)M + off;
        for (int64_t i = 0; i < per; ++i) dst[i] = fp8_from_float(src[i]);
      }
    }
  return 0;
}

static double load_elem(const void* M, int dtype, int64_t pos) {
  if (dtype == 0) return (double)((const float*)M)[pos];
  if (dtype == 1) return bf16_to_double(((const uint16_t*)M)[pos]);
  return fp8_to_double(((const uint8_t*)M)[pos]);
}

static void store_elem(void* M, int dtype, int64_t pos, double val) {
  if (dtype == 0) ((float*)M)[pos] = (float)val;
  else ((uint16_t*)M)[pos] = bf16_from_double(val);
}

/* T sequential steps on ONE memory M [N, d_v].  Per step t: the gated delta
 * write of rows widx[t, 0..W) with weights wk, then the read of rows
 * ridx[t, 0..R) with weights rw into out[t, :].  Only columns [c0, c1) are
 * computed (each column's recurrence involves that column alone); out's other
 * columns are left untouched.  v, out [T, d_v]; alpha, beta [T]. */
int oracle_scan(void* M, int dtype, int64_t N, int d_v, int64_t T, int W, int R,
                const int32_t* widx, const double* wk, const int32_t* ridx, const double* rw,
                const float* v, const float* alpha, const float* beta, float* out, int c0,
                int c1) {
  if (!M || !widx || !wk || !ridx || !rw || !v || !alpha || !beta || !out)
    return fail("null pointer");
  if (N < 1 || d_v < 1 || T < 0 || W < 1 || R < 1 || dtype < 0 || dtype > 2)
    return fail("bad sizes");
  if (c0 < 0 || c1 > d_v || c0 > c1) return fail("bad column range");
  for (int64_t t = 0; t < T; ++t) {
    const int32_t* wi = widx + t * W;
    const int32_t* ri = ridx + t * R;
    for (int j = 0; j < W; ++j) {
      if (wi[j] < 0 || wi[j] >= N) return fail("write index out of range");
      for (int l = 0; l < j; ++l)
        if (wi[l] == wi[j]) return fail("write indices of a step must be distinct");
    }
    for (int j = 0; j < R; ++j)
      if (ri[j] < 0 || ri[j] >= N) return fail("read index out of range");
    const float* vt = v + t * d_v;
    if (!all_finite(vt, d_v) || !isfinite(alpha[t]) || !isfinite(beta[t]))
      return fail("non-finite v/alpha/beta");
    double a = (double)alpha[t], be = (double)beta[t];
    /* write: forget gate then delta update, selected rows only */
    for (int j = 0; j < W; ++j) {
      int64_t row = (int64_t)wi[j] * d_v;
      double k = wk[t * W + j];
      for (int c = c0; c < c1; ++c) {
        double m = load_elem(M, dtype, row + c);
        if (dtype == 2) {
          /* fp8 state: the stored code is decided by the binary32 update,
           * taken in this order -- Mt = alpha*m; d = v - Mt;
           * u = fma(beta*k, d, Mt) -- with each operation rounded to
           * binary32, then rounded once more to E4M3.  The weight k must be
           * a binary32 value for this to be the same computation on any
           * implementation. */
          float mt = (float)alpha[t] * (float)m;
          float d = vt[c] - mt;
          float g = beta[t] * (float)k;
          ((uint8_t*)M)[row + c] = fp8_from_float(fmaf(g, d, mt));
          continue;
        }
        double mt = a * m;
        double u = mt + be * k * ((double)vt[c] - mt);
        store_elem(M, dtype, row + c, u);
      }
    }
    /* read: weighted sum of the stored rows after the write */
    for (int c = c0; c < c1; ++c) {
      double acc = 0.0;
      for (int j = 0; j < R; ++j)
        acc += rw[t * R + j] * load_elem(M, dtype, (int64_t)ri[j] * d_v + c);
      out[t * d_v + c] = (float)acc;
    }
  }
  return 0;
}

/* One single-token step for every (b,h): write and read selections from the
 * halves, then the write and the read, on M [B,H,N,d_v].  s1, s2, q1, q2
 * [B,H,n]; v, out [B,H,d_v]; alpha, beta [B,H]; widx [B,H,W], ridx [B,H,R]
 * (may be NULL). */
int oracle_step_decode(void* M, int dtype, int B, int H, int n, int d_v, int W, int R,
                       const float* s1, const float* s2, const float* q1, const float* q2,
                       const float* v, const float* alpha, const float* beta, float* out,
                       int32_t* widx, int32_t* ridx) {
  if (B < 1 || H < 1 || n < 1 || W < 1 || R < 1 || W > n || R > n || dtype < 0 || dtype > 2)
    return fail("bad sizes");
  int64_t N = (int64_t)n * n;
  int32_t* wi = (int32_t*)malloc(sizeof(int32_t) * (size_t)W);
  int32_t* ri = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
  double* wk = (double*)malloc(sizeof(double) * (size_t)W);
  double* rw = (double*)malloc(sizeof(double) * (size_t)R);
  int rc = (wi && ri && wk && rw) ? 0 : fail("out of memory");
  for (int64_t u = 0; rc == 0 && u < (int64_t)B * H; ++u) {
    rc = oracle_select(s1 + u * n, s2 + u * n, 1, n, W, wi, NULL, wk);
    if (rc == 0) rc = oracle_select(q1 + u * n, q2 + u * n, 1, n, R, ri, NULL, rw);
    if (rc != 0) break;
    /* bytes per state element: fp32 4, bf16 2, fp8 E4M3 1 */
    size_t es = dtype == 0 ? sizeof(float) : (dtype == 1 ? sizeof(uint16_t) : sizeof(uint8_t));
    void* Mu = (char*)M + (size_t)u * (size_t)N * (size_t)d_v * es;
    rc = oracle_scan(Mu, dtype, N, d_v, 1, W, R, wi, wk, ri, rw, v + u * d_v, alpha + u,
                     beta + u, out + u * d_v, 0, d_v);
    if (rc == 0 && widx) memcpy(widx + u * W, wi, sizeof(int32_t) * (size_t)W);
    if (rc == 0 && ridx) memcpy(ridx + u * R, ri, sizeof(int32_t) * (size_t)R);
  }
  free(wi); free(ri); free(wk); free(rw);
  return rc;
}

/* ------------------------------------------------------------ projections
 *
 * The step's inputs come from linear projections of each token ("Riepilogo
 * Tecnico: Sparse Delta Memory (SDM)", section "Meccanismo Core", item 2: the
 * projected keys and queries are split in two halves; section "Design
 * IsoFLOP": the projections are sized like the baseline's).  Per token x
 * (d_model values, bf16) and head h, y = W_h x with W_h [P, d_model] bf16,
 * P = 4n + d_v + 2, rows in this order: the key halves s1, s2, the query
 * halves q1, q2 (n each), v (d_v), then the two gate pre-activations.  The
 * pages name the gates alpha_t, beta_t but not how they are formed; here
 * alpha = sigma(y_alpha), beta = sigma(y_beta) with the logistic sigma, which
 * keeps both in (0, 1).
 *
 * X [M, d_model] and Wt [H, P, d_model] are bf16 bits.  Outputs, for token
 * m (= b*T + t): y [M, H, P] double (the exact dot products: every product of
 * two bf16 values is exact in double, and the sum is taken in order), and
 * yabs [M, H, P] double, the sum of |x_k w_k| (for the rounding bound of a
 * binary32 accumulation).  The gates are not applied here; oracle_sigmoid()
 * gives them. */
static double bf16_bits_to_double(uint16_t h) { return bf16_to_double(h); }

int oracle_project(const uint16_t* X, const uint16_t* Wt, int64_t M, int d_model, int H, int P,
                   double* y, double* yabs) {
  if (!X || !Wt || !y || !yabs) return fail("null pointer");
  if (M < 0 || d_model < 1 || H < 1 || P < 1) return fail("bad sizes");
  for (int64_t m = 0; m < M; ++m)
    for (int h = 0; h < H; ++h)
      for (int p = 0; p < P; ++p) {
        const uint16_t* w = Wt + ((int64_t)h * P + p) * d_model;
        const uint16_t* x = X + m * d_model;
        double acc = 0.0, aabs = 0.0;
        for (int k = 0; k < d_model; ++k) {
          double prod = bf16_bits_to_double(x[k]) * bf16_bits_to_double(w[k]);
          acc += prod;
          aabs += fabs(prod);
        }
        y[(m * H + h) * P + p] = acc;
        yabs[(m * H + h) * P + p] = aabs;
      }
  return 0;
}

double oracle_sigmoid(double y) { return 1.0 / (1.0 + exp(-y)); }

/* ------------------------------------------------------------- backward
 *
 * Gradients of the step for training.  The pages train the whole layer end to
 * end and learn M0 ("Stato Iniziale Appreso"; "学習された初期状態"), so the
 * reverse pass below differentiates the write and read of "Meccanismo Core"
 * items 3 and 4 with the selections held fixed (the chosen slot indices are
 * piecewise constant in the scores; gradients reach the scores only through
 * the selection weights).  fp32 state only.
 *
 * Forward of one step, per write row i = f_j with pre-write stored row P:
 *   u = alpha*P + (beta*k_j)*(v - alpha*P)  = alpha*(1 - beta*k_j)*P + beta*k_j*v
 * and the read o = sum_j r_j * M_t[g_j] of the stored rows after the write.
 * With G the gradient of the loss with respect to the memory after step t,
 * the chain rule gives, in reverse time order:
 *   read:   dr_j = <do_t, M_t[g_j]>;  G[g_j] += r_j * do_t
 *   write:  with g = G[f_j] (already holding this step's read part):
 *           dv_t += beta*k_j * g
 *           dalpha_t += <g, P> * (1 - beta*k_j)
 *           d(beta k_j) = <g, v_t - alpha*P>;  dk_j = beta * d(beta k_j);
 *           dbeta_t += k_j * d(beta k_j)
 *           G[f_j] = alpha*(1 - beta*k_j) * g        (the row's own carry)
 *   then the rows are restored to P, giving the memory after step t-1.
 * Rows not written at step t carry G unchanged (the unselected rows are left
 * as they were).  After t = 0, G is the gradient with respect to the memory's
 * initial state.  All arithmetic in double; the forward replay stores fp32
 * rows exactly as oracle_scan does. */

/* One memory.  M0 [N,d_v] fp32: the memory before step 0.  G [N,d_v] double:
 * in, the gradient with respect to the memory after step T-1; out, with
 * respect to M0.  dout, dv [T,d_v]; dwk [T,W]; drw [T,R]; dalpha, dbeta [T].
 * tape [T,W,d_v] (may be NULL): the pre-write rows of every step.  rtape
 * [T,R,d_v] (may be NULL): the rows every step's read saw (after its write).
 * MT [N,d_v] (may be NULL): the memory after step T-1. */
int oracle_scan_backward(const float* M0, int64_t N, int d_v, int64_t T, int W, int R,
                         const int32_t* widx, const double* wk, const int32_t* ridx,
                         const double* rw, const float* v, const float* alpha,
                         const float* beta, const float* dout, double* G, double* dv,
                         double* dwk, double* drw, double* dalpha, double* dbeta, float* tape,
                         float* rtape, float* MT) {
  if (!M0 || !widx || !wk || !ridx || !rw || !v || !alpha || !beta || !dout || !G || !dv ||
      !dwk || !drw || !dalpha || !dbeta)
    return fail("null pointer");
  if (N < 1 || d_v < 1 || T < 0 || W < 1 || R < 1) return fail("bad sizes");
  if (!all_finite(dout, T * d_v)) return fail("non-finite output gradient");
  for (int64_t t = 0; t < T; ++t) {
    for (int j = 0; j < W; ++j) {
      int32_t r = widx[t * W + j];
      if (r < 0 || r >= N) return fail("write index out of range");
      for (int l = 0; l < j; ++l)
        if (widx[t * W + l] == r) return fail("write indices of a step must be distinct");
    }
    for (int j = 0; j < R; ++j) {
      int32_t r = ridx[t * R + j];
      if (r < 0 || r >= N) return fail("read index out of range");
      for (int l = 0; l < j; ++l)
        if (ridx[t * R + l] == r) return fail("read indices of a step must be distinct");
    }
  }
  float* M = (float*)malloc(sizeof(float) * (size_t)(N * d_v));
  float* P = (float*)malloc(sizeof(float) * (size_t)(T * W * d_v + 1));
  if (!M || !P) {
    free(M); free(P);
    return fail("out of memory");
  }
  memcpy(M, M0, sizeof(float) * (size_t)(N * d_v));
  /* forward replay, keeping every step's pre-write rows */
  for (int64_t t = 0; t < T; ++t) {
    double a = (double)alpha[t], be = (double)beta[t];
    for (int j = 0; j < W; ++j) {
      float* row = M + (int64_t)widx[t * W + j] * d_v;
      float* keep = P + (t * W + j) * d_v;
      double k = wk[t * W + j];
      for (int c = 0; c < d_v; ++c) {
        keep[c] = row[c];
        double mt = a * (double)row[c];
        row[c] = (float)(mt + be * k * ((double)v[t * d_v + c] - mt));
      }
    }
  }
  if (MT) memcpy(MT, M, sizeof(float) * (size_t)(N * d_v));
  if (tape) memcpy(tape, P, sizeof(float) * (size_t)(T * W * d_v));
  /* reverse pass */
  for (int64_t t = T - 1; t >= 0; --t) {
    const float* dot = dout + t * d_v;
    double a = (double)alpha[t], be = (double)beta[t];
    for (int j = 0; j < R; ++j) {
      const float* row = M + (int64_t)ridx[t * R + j] * d_v;
      double s = 0.0;
      for (int c = 0; c < d_v; ++c) s += (double)dot[c] * (double)row[c];
      drw[t * R + j] = s;
      if (rtape) memcpy(rtape + (t * R + j) * d_v, row, sizeof(float) * (size_t)d_v);
    }
    for (int j = 0; j < R; ++j) {
      double* g = G + (int64_t)ridx[t * R + j] * d_v;
      for (int c = 0; c < d_v; ++c) g[c] += rw[t * R + j] * (double)dot[c];
    }
    for (int c = 0; c < d_v; ++c) dv[t * d_v + c] = 0.0;
    double da = 0.0, db = 0.0;
    for (int j = 0; j < W; ++j) {
      double* g = G + (int64_t)widx[t * W + j] * d_v;
      const float* keep = P + (t * W + j) * d_v;
      double k = wk[t * W + j], bk = be * k;
      double dbk = 0.0, gp = 0.0;
      for (int c = 0; c < d_v; ++c) {
        dv[t * d_v + c] += bk * g[c];
        gp += g[c] * (double)keep[c];
        dbk += g[c] * ((double)v[t * d_v + c] - a * (double)keep[c]);
        g[c] = a * (1.0 - bk) * g[c];
      }
      da += gp * (1.0 - bk);
      dwk[t * W + j] = be * dbk;
      db += k * dbk;
    }
    dalpha[t] = da;
    dbeta[t] = db;
    for (int j = 0; j < W; ++j)
      memcpy(M + (int64_t)widx[t * W + j] * d_v, P + (t * W + j) * d_v, sizeof(float) * (size_t)d_v);
  }
  free(M);
  free(P);
  return 0;
}

/* Gradient through the selection weights to the half scores, selections held
 * fixed.  The weights are the softmax of the selected sums sigma_j, and
 * sigma_j = x1[a_j] + x2[b_j] with f_j = a_j*n + b_j, so
 *   dsigma_j = w_j * (dw_j - sum_l w_l dw_l),
 *   dx1[a] = sum of dsigma_j over j with a_j = a, dx2[b] likewise,
 * and zero for every half index that no selected slot uses.
 * idx, w, dw [units, K]; dx1, dx2 [units, n]. */
int oracle_select_backward(const int32_t* idx, const double* w, const double* dw, int64_t units,
                           int n, int K, double* dx1, double* dx2) {
  if (!idx || !w || !dw || !dx1 || !dx2) return fail("null pointer");
  if (units < 0 || n < 1 || K < 1 || K > n) return fail("bad sizes");
  for (int64_t u = 0; u < units; ++u) {
    const int32_t* f = idx + u * K;
    double s = 0.0;
    for (int j = 0; j < K; ++j) s += w[u * K + j] * dw[u * K + j];
    for (int i = 0; i < n; ++i) dx1[u * n + i] = dx2[u * n + i] = 0.0;
    for (int j = 0; j < K; ++j) {
      if (f[j] < 0 || f[j] >= n * n) return fail("slot index out of range");
      double ds = w[u * K + j] * (dw[u * K + j] - s);
      dx1[u * n + f[j] / n] += ds;
      dx2[u * n + f[j] % n] += ds;
    }
  }
  return 0;
}

/* bf16 and fp8 helpers exposed for the tests of the oracle itself. */
uint16_t oracle_bf16_from_double(double x) { return bf16_from_double(x); }
double oracle_bf16_to_double(uint16_t h) { return bf16_to_double(h); }
uint8_t oracle_fp8_from_float(float x) { return fp8_from_float(x); }
double oracle_fp8_to_double(uint8_t c) { return fp8_to_double(c); }
