// C-ABI entry points of libsdm.so: argument validation (before any launch),
// dispatch to the kernels, HIP error mapping and the per-thread error text.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/sdm.h"
#include "internal.h"
#include "planned.h"
#include "ranges.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

bool debug_sync() {
  static const int on = [] {
    const char* e = getenv("SDM_DEBUG_SYNC");
    return (e && e[0] == '1') ? 1 : 0;
  }();
  return on != 0;
}

int finish(const char* what, hipError_t launch_err, hipStream_t stream) {
  if (launch_err != hipSuccess)
    return fail(SDM_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(launch_err));
  if (debug_sync()) {
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
      return fail(SDM_ERR_HIP, "%s: kernel failed: %s", what, hipGetErrorString(e));
  }
  g_err[0] = '\0';
  return SDM_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool n_supported(int n) {
  return (n >= 1 && n <= 64) || n == 128 || n == 256 || n == 512 || n == 1024 || n == 2048;
}

bool dv_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

int check_n_k(int n, int K, const char* kname) {
  if (n < 1) return fail(SDM_ERR_INVALID, "n must be >= 1 (got %d)", n);
  if (K < 1 || K > n) return fail(SDM_ERR_INVALID, "%s must be in [1, n] (got %s=%d, n=%d)",
                                  kname, kname, K, n);
  if (!n_supported(n))
    return fail(SDM_ERR_UNSUPPORTED, "n=%d not compiled (1..64 or 128..2048 powers of two)", n);
  if (K > 64) return fail(SDM_ERR_UNSUPPORTED, "%s=%d > 64 not compiled", kname, K);
  return SDM_OK;
}

int check_scores(const float* p, int n, const char* name) {
  if (!p) return fail(SDM_ERR_INVALID, "%s is NULL", name);
  size_t a = n >= 256 ? 16 : 4;
  if (!aligned(p, a)) return fail(SDM_ERR_INVALID, "%s must be %zu-byte aligned", name, a);
  return SDM_OK;
}

int check_state(const void* M, int dtype, int64_t N, int d_v) {
  if (!M) return fail(SDM_ERR_INVALID, "M is NULL");
  if (!aligned(M, 16)) return fail(SDM_ERR_INVALID, "M must be 16-byte aligned");
  if (dtype != SDM_F32 && dtype != SDM_BF16 && dtype != SDM_FP8)
    return fail(SDM_ERR_INVALID, "dtype must be SDM_F32, SDM_BF16 or SDM_FP8 (got %d)", dtype);
  if (N < 1 || N >= ((int64_t)1 << 31))
    return fail(SDM_ERR_INVALID, "N must be in [1, 2^31) (got %lld)", (long long)N);
  if (d_v < 1) return fail(SDM_ERR_INVALID, "d_v must be >= 1 (got %d)", d_v);
  if (!dv_supported(d_v))
    return fail(SDM_ERR_UNSUPPORTED, "d_v=%d not compiled (16, 32, 64, 128, 256)", d_v);
  if (dtype == SDM_FP8 && d_v < 32)
    return fail(SDM_ERR_UNSUPPORTED, "fp8 state needs d_v >= 32 (got %d)", d_v);
  return SDM_OK;
}

int64_t elem_bytes(int dtype) { return dtype == SDM_F32 ? 4 : (dtype == SDM_BF16 ? 2 : 1); }

}  // namespace

extern "C" {

int sdm_abi_version(void) { return 6; }

const char* sdm_status_string(int status) {
  switch (status) {
    case SDM_OK: return "SDM_OK";
    case SDM_ERR_INVALID: return "SDM_ERR_INVALID";
    case SDM_ERR_UNSUPPORTED: return "SDM_ERR_UNSUPPORTED";
    case SDM_ERR_HIP: return "SDM_ERR_HIP";
    default: return "unknown status";
  }
}

const char* sdm_last_error(void) { return g_err; }

int sdm_project(const uint16_t* X, const uint16_t* Wt, int B, int T, int d_model, int H, int n,
                int d_v, float* s1, float* s2, float* q1, float* q2, float* v, float* alpha,
                float* beta, void* stream) {
  if (B < 0 || T < 0) return fail(SDM_ERR_INVALID, "B and T must be >= 0 (got %d, %d)", B, T);
  if (H < 1 || n < 1 || d_v < 1)
    return fail(SDM_ERR_INVALID, "H, n and d_v must be >= 1 (got %d, %d, %d)", H, n, d_v);
  if (d_model < 64 || d_model > 65536 || d_model % 64 != 0)
    return fail(SDM_ERR_UNSUPPORTED, "d_model must be a multiple of 64 in [64, 65536] (got %d)",
                d_model);
  const int64_t P = 4 * (int64_t)n + d_v + 2, cols = (int64_t)H * P, M = (int64_t)B * T;
  if (cols >= ((int64_t)1 << 31))
    return fail(SDM_ERR_UNSUPPORTED, "H*(4n + d_v + 2) must be below 2^31 (got %lld)",
                (long long)cols);
  if (M == 0) return finish("sdm_project", hipSuccess, (hipStream_t)stream);  // arrays may be NULL
  if (sdm::project_blocks(M, cols) > sdm::kMaxStrideBlocks)
    return fail(SDM_ERR_UNSUPPORTED, "more than 2^24 - 1 output tiles of 256 x 256 (B*T=%lld, "
                "H*P=%lld); split the tokens over several calls", (long long)M, (long long)cols);
  if (!X || !Wt) return fail(SDM_ERR_INVALID, "X and Wt must not be NULL");
  if (!aligned(X, 16) || !aligned(Wt, 16))
    return fail(SDM_ERR_INVALID, "X and Wt must be 16-byte aligned");
  float* outs[7] = {s1, s2, q1, q2, v, alpha, beta};
  const char* names[7] = {"s1", "s2", "q1", "q2", "v", "alpha", "beta"};
  for (int i = 0; i < 7; ++i) {
    if (!outs[i]) return fail(SDM_ERR_INVALID, "%s is NULL", names[i]);
    if (!aligned(outs[i], 4)) return fail(SDM_ERR_INVALID, "%s must be 4-byte aligned", names[i]);
  }
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_project", sdm::launch_project(X, Wt, B, T, d_model, H, n, d_v, s1, s2, q1, q2,
                                                   v, alpha, beta, s), s);
}

int sdm_select(const float* x1, const float* x2, int64_t units, int n, int K, int32_t* idx,
               float* score, float* weight, void* stream) {
  int rc;
  if (units < 0) return fail(SDM_ERR_INVALID, "units must be >= 0");
  if ((rc = check_n_k(n, K, "K"))) return rc;
  if (units == 0) return finish("sdm_select", hipSuccess, (hipStream_t)stream);  // arrays may be NULL
  if ((rc = check_scores(x1, n, "x1")) || (rc = check_scores(x2, n, "x2"))) return rc;
  if (!idx || !weight) return fail(SDM_ERR_INVALID, "idx and weight must not be NULL");
  if (units > sdm::kMaxWaveUnits)
    return fail(SDM_ERR_UNSUPPORTED, "units must be at most 2^26 - 4 per call (got %lld)",
                (long long)units);
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_select", sdm::launch_select(x1, x2, units, n, K, idx, score, weight, s), s);
}

int sdm_state_init(void* M, int dtype, const float* M0, int B, int H, int64_t N, int d_v,
                   void* stream) {
  int rc;
  if ((rc = check_state(M, dtype, N, d_v))) return rc;
  if (!M0) return fail(SDM_ERR_INVALID, "M0 is NULL");
  if (!aligned(M0, 16)) return fail(SDM_ERR_INVALID, "M0 must be 16-byte aligned");
  if (B < 1 || H < 1) return fail(SDM_ERR_INVALID, "B and H must be >= 1");
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_state_init", sdm::launch_state_init(M, dtype, M0, B, H, N, d_v, s), s);
}

}  // extern "C"

namespace {

int check_scan_args(const void* M, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W,
                    int R, const int32_t* widx, const float* wk, const int32_t* ridx,
                    const float* rw, const float* v, const float* alpha, const float* beta,
                    const float* out) {
  int rc;
  if ((rc = check_state(M, dtype, N, d_v))) return rc;
  if (T < 0) return fail(SDM_ERR_INVALID, "T must be >= 0");
  // with T = 0 every per-step array is empty and may be NULL
  if (T > 0 && (!widx || !wk || !ridx || !rw || !v || !alpha || !beta || !out))
    return fail(SDM_ERR_INVALID, "a scan input or output pointer is NULL");
  if (!aligned(v, 16) || !aligned(out, 16))
    return fail(SDM_ERR_INVALID, "v and out must be 16-byte aligned");
  if (!aligned(widx, 4) || !aligned(wk, 4) || !aligned(ridx, 4) || !aligned(rw, 4) ||
      !aligned(alpha, 4) || !aligned(beta, 4))
    return fail(SDM_ERR_INVALID, "index, weight and gate arrays must be 4-byte aligned");
  if (B < 1 || H < 1) return fail(SDM_ERR_INVALID, "B and H must be >= 1");
  if ((int64_t)B * H > sdm::kMaxMemories)
    return fail(SDM_ERR_UNSUPPORTED, "B*H must be at most 2^20 memories per call");
  // bounds every size product the call and its launchers form from T (e.g.
  // B*H*T*d_v*4 bytes of output, T*(W+R)*d_v*4 bytes of tape) well inside 63 bits
  if (T > sdm::kMaxSteps || (int64_t)B * H * T > sdm::kMaxMemorySteps)
    return fail(SDM_ERR_UNSUPPORTED, "T must be at most 2^32 and B*H*T at most 2^40 per call");
  if (W < 1 || R < 1) return fail(SDM_ERR_INVALID, "W and R must be >= 1");
  if (W > 64 || R > 64) return fail(SDM_ERR_UNSUPPORTED, "W and R above 64 are not compiled");
  if (W > N || R > N) return fail(SDM_ERR_INVALID, "W and R must not exceed N");
  if (N * d_v * elem_bytes(dtype) >= ((int64_t)1 << 31))
    return fail(SDM_ERR_UNSUPPORTED, "one memory's table must be below 2 GiB for sdm_scan");
  if (!sdm::ranges::scan_ok(N, d_v, (int)elem_bytes(dtype), T, W, R, false))
    return fail(SDM_ERR_UNSUPPORTED, "a state tile's buffer range does not fit 31 bits");
  return SDM_OK;
}

}  // namespace

extern "C" {

int sdm_scan(void* M, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
             const int32_t* widx, const float* wk, const int32_t* ridx, const float* rw,
             const float* v, const float* alpha, const float* beta, float* out, void* stream) {
  int rc;
  if ((rc = check_scan_args(M, dtype, B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta,
                            out)))
    return rc;
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_scan",
                sdm::launch_scan(M, dtype, B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha,
                                 beta, out, nullptr, s),
                s);
}

int sdm_scan_train(void* M, int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                   const int32_t* widx, const float* wk, const int32_t* ridx, const float* rw,
                   const float* v, const float* alpha, const float* beta, float* out,
                   float* tape, void* stream) {
  int rc;
  if ((rc = check_scan_args(M, SDM_F32, B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha,
                            beta, out)))
    return rc;
  if (T > 0 && !tape) return fail(SDM_ERR_INVALID, "tape is NULL");
  if (!aligned(tape, 16)) return fail(SDM_ERR_INVALID, "tape must be 16-byte aligned");
  if (T * (W + R) * d_v * 4 >= ((int64_t)1 << 31))
    return fail(SDM_ERR_UNSUPPORTED, "one memory's tape (T*(W+R)*d_v*4 bytes) must be below 2 GiB; "
                "split the sequence into consecutive calls");
  if (!sdm::ranges::scan_ok(N, d_v, 4, T, W, R, true))
    return fail(SDM_ERR_UNSUPPORTED, "a state or tape tile's buffer range does not fit 31 bits");
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_scan_train",
                sdm::launch_scan(M, SDM_F32, B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha,
                                 beta, out, tape, s),
                s);
}

size_t sdm_scan_backward_workspace_size(int B, int H, int d_v, int64_t T, int W, int R) {
  if (B < 1 || H < 1 || T < 0 || W < 1 || R < 1 || !dv_supported(d_v)) return 0;
  return sdm::scan_backward_workspace_bytes(B * H, d_v, T, W, R);
}

}  // extern "C"

namespace {

// Validation shared by sdm_scan_backward and sdm_scan_backward_noalloc; on
// success *need is the workspace the reverse pass uses, in bytes.
int check_backward_args(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                        const int32_t* widx, const float* wk, const int32_t* ridx,
                        const float* rw, const float* v, const float* alpha, const float* beta,
                        const float* tape, const float* dout, float* G, float* dv, float* dwk,
                        float* drw, float* dalpha, float* dbeta, const uint64_t* first,
                        size_t* need) {
  int rc;
  // G has the state's shape and type: it stands for the state in the shared checks
  if ((rc = check_scan_args(G, SDM_F32, B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha,
                            beta, dv)))
    return rc;
  if (T > 0 && (!tape || !dout || !dwk || !drw || !dalpha || !dbeta))
    return fail(SDM_ERR_INVALID, "a backward input or output pointer is NULL");
  if (!aligned(tape, 16) || !aligned(dout, 16) || !aligned(G, 16))
    return fail(SDM_ERR_INVALID, "tape, dout and G must be 16-byte aligned");
  if (!aligned(dwk, 4) || !aligned(drw, 4) || !aligned(dalpha, 4) || !aligned(dbeta, 4))
    return fail(SDM_ERR_INVALID, "dwk, drw, dalpha and dbeta must be 4-byte aligned");
  if (!aligned(first, 8)) return fail(SDM_ERR_INVALID, "first must be 8-byte aligned");
  if (T >= ((int64_t)1 << 26)) return fail(SDM_ERR_UNSUPPORTED, "T must be below 2^26");
  if ((int64_t)B * H * T > sdm::kMaxWaveUnits)
    return fail(SDM_ERR_UNSUPPORTED,
                "B*H*T must be at most 2^26 - 4 (one finishing wavefront per memory and step)");
  if (T * (W + R) * d_v * 4 >= ((int64_t)1 << 31))
    return fail(SDM_ERR_UNSUPPORTED, "one memory's tape (T*(W+R)*d_v*4 bytes) must be below 2 GiB; "
                "split the sequence into consecutive calls");
  if (!sdm::ranges::scan_backward_ok(N, d_v, T, W, R))
    return fail(SDM_ERR_UNSUPPORTED, "a gradient or tape tile's buffer range does not fit 31 bits");
  *need = sdm::scan_backward_workspace_bytes(B * H, d_v, T, W, R);
  return SDM_OK;
}

}  // namespace

extern "C" {

int sdm_scan_backward(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                      const int32_t* widx, const float* wk, const int32_t* ridx,
                      const float* rw, const float* v, const float* alpha, const float* beta,
                      const float* tape, const float* dout, float* G, float* dv, float* dwk,
                      float* drw, float* dalpha, float* dbeta, const uint64_t* first,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  size_t need = 0;
  if ((rc = check_backward_args(B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta, tape,
                                dout, G, dv, dwk, drw, dalpha, dbeta, first, &need)))
    return rc;
  if (T > 0 && !workspace) return fail(SDM_ERR_INVALID, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(SDM_ERR_INVALID, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(SDM_ERR_INVALID, "workspace of %zu bytes is below the %zu required",
                workspace_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_scan_backward",
                sdm::launch_scan_backward(B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha,
                                          beta, tape, dout, G, dv, dwk, drw, dalpha, dbeta, first,
                                          reinterpret_cast<float*>(workspace), s),
                s);
}

int sdm_scan_backward_noalloc(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                              const int32_t* widx, const float* wk, const int32_t* ridx,
                              const float* rw, const float* v, const float* alpha,
                              const float* beta, const float* tape, const float* dout, float* G,
                              float* dv, float* dwk, float* drw, float* dalpha, float* dbeta,
                              const uint64_t* first, void* stream) {
  int rc;
  size_t need = 0;
  if ((rc = check_backward_args(B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha, beta, tape,
                                dout, G, dv, dwk, drw, dalpha, dbeta, first, &need)))
    return rc;
  if (need > sdm::kStaticScratchBytes)
    return fail(SDM_ERR_UNSUPPORTED,
                "the reverse pass needs %zu bytes of workspace, above the library's %zu-byte "
                "static buffer; use sdm_scan_backward with a caller workspace",
                need, sdm::kStaticScratchBytes);
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) return finish("sdm_scan_backward_noalloc", hipSuccess, s);
  void* ws = nullptr;
  const hipError_t e = sdm::static_scratch(&ws);
  if (e != hipSuccess)
    return fail(SDM_ERR_HIP, "sdm_scan_backward_noalloc: device scratch lookup failed: %s",
                hipGetErrorString(e));
  return finish("sdm_scan_backward_noalloc",
                sdm::launch_scan_backward(B, H, N, d_v, T, W, R, widx, wk, ridx, rw, v, alpha,
                                          beta, tape, dout, G, dv, dwk, drw, dalpha, dbeta, first,
                                          reinterpret_cast<float*>(ws), s),
                s);
}

int sdm_select_backward(const int32_t* idx, const float* weight, const float* dweight,
                        int64_t units, int n, int K, float* dx1, float* dx2, void* stream) {
  int rc;
  if (units < 0) return fail(SDM_ERR_INVALID, "units must be >= 0");
  if ((rc = check_n_k(n, K, "K"))) return rc;
  if (units == 0)  // the arrays are empty and may be NULL
    return finish("sdm_select_backward", hipSuccess, (hipStream_t)stream);
  if (!idx || !weight || !dweight || !dx1 || !dx2)
    return fail(SDM_ERR_INVALID, "a selection-gradient pointer is NULL");
  if (!aligned(idx, 4) || !aligned(weight, 4) || !aligned(dweight, 4) || !aligned(dx1, 4) ||
      !aligned(dx2, 4))
    return fail(SDM_ERR_INVALID, "selection-gradient arrays must be 4-byte aligned");
  if (units > sdm::kMaxWaveUnits)
    return fail(SDM_ERR_UNSUPPORTED, "units must be at most 2^26 - 4 per call (got %lld)",
                (long long)units);
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_select_backward",
                sdm::launch_select_backward(idx, weight, dweight, units, n, K, dx1, dx2, s), s);
}

int sdm_state_init_backward(const float* G, int B, int H, int64_t N, int d_v,
                            const uint32_t* seen, float* dM0, void* stream) {
  int rc;
  if ((rc = check_state(G, SDM_F32, N, d_v))) return rc;
  if (!dM0) return fail(SDM_ERR_INVALID, "dM0 is NULL");
  if (!aligned(dM0, 16)) return fail(SDM_ERR_INVALID, "dM0 must be 16-byte aligned");
  if (!aligned(seen, 4)) return fail(SDM_ERR_INVALID, "seen must be 4-byte aligned");
  if (B < 1 || H < 1) return fail(SDM_ERR_INVALID, "B and H must be >= 1");
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_state_init_backward",
                sdm::launch_state_init_backward(G, B, H, N, d_v, seen, dM0, s), s);
}

int sdm_touch_prepare(int B, int H, int64_t N, int64_t T, int W, int R, const int32_t* widx,
                      const int32_t* ridx, uint32_t* seen, uint64_t* first, void* stream) {
  if (B < 1 || H < 1) return fail(SDM_ERR_INVALID, "B and H must be >= 1");
  if ((int64_t)B * H > sdm::kMaxMemories)
    return fail(SDM_ERR_UNSUPPORTED, "B*H must be at most 2^20 memories per call");
  if (N < 1) return fail(SDM_ERR_INVALID, "N must be >= 1");
  if (N > sdm::kTouchMaxN)
    return fail(SDM_ERR_UNSUPPORTED, "N must be at most 2^20 (one N-bit table per memory in LDS)");
  if (W < 1 || W > 64 || R < 1 || R > 64) return fail(SDM_ERR_INVALID, "W and R must be in [1, 64]");
  if (T < 0) return fail(SDM_ERR_INVALID, "T must be >= 0");
  if (T >= ((int64_t)1 << 26)) return fail(SDM_ERR_UNSUPPORTED, "T must be below 2^26");
  if (T * (W > R ? W : R) * 4 >= ((int64_t)1 << 31))
    return fail(SDM_ERR_UNSUPPORTED, "one memory's index arrays must be below 2 GiB");
  if (!seen) return fail(SDM_ERR_INVALID, "seen is NULL");
  if (T > 0 && (!widx || !ridx || !first))
    return fail(SDM_ERR_INVALID, "widx, ridx and first must not be NULL");
  if (!aligned(seen, 4) || !aligned(widx, 4) || !aligned(ridx, 4) || !aligned(first, 8))
    return fail(SDM_ERR_INVALID, "index arrays and seen must be 4-byte, first 8-byte aligned");
  if (!sdm::ranges::touch_ok(T, W, R))
    return fail(SDM_ERR_UNSUPPORTED, "an index or mask buffer range does not fit 31 bits");
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_touch_prepare",
                sdm::launch_touch_prepare(B, H, N, T, W, R, widx, ridx, seen, first, s), s);
}

int sdm_step_decode(void* M, int dtype, int B, int H, int n, int d_v, int W, int R,
                    const float* s1, const float* s2, const float* q1, const float* q2,
                    const float* v, const float* alpha, const float* beta, float* out,
                    int32_t* widx, int32_t* ridx, void* stream) {
  int rc;
  if ((rc = check_n_k(n, W, "W")) || (rc = check_n_k(n, R, "R"))) return rc;
  if ((rc = check_state(M, dtype, (int64_t)n * n, d_v))) return rc;
  if (dtype == SDM_FP8)
    return fail(SDM_ERR_UNSUPPORTED, "sdm_step_decode supports fp32 and bf16 state");
  if ((rc = check_scores(s1, n, "s1")) || (rc = check_scores(s2, n, "s2")) ||
      (rc = check_scores(q1, n, "q1")) || (rc = check_scores(q2, n, "q2")))
    return rc;
  if (!v || !alpha || !beta || !out)
    return fail(SDM_ERR_INVALID, "v, alpha, beta and out must not be NULL");
  if (!aligned(v, 16) || !aligned(out, 4) || !aligned(alpha, 4) || !aligned(beta, 4))
    return fail(SDM_ERR_INVALID, "v must be 16-byte aligned; out, alpha, beta 4-byte");
  if ((widx && !aligned(widx, 4)) || (ridx && !aligned(ridx, 4)))
    return fail(SDM_ERR_INVALID, "widx and ridx must be 4-byte aligned");
  if (B < 1 || H < 1) return fail(SDM_ERR_INVALID, "B and H must be >= 1");
  if ((int64_t)B * H > sdm::kMaxMemories)
    return fail(SDM_ERR_UNSUPPORTED, "B*H must be at most 2^20 memories per call");
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_step_decode",
                sdm::launch_step_decode(M, dtype, B, H, n, d_v, W, R, s1, s2, q1, q2, v, alpha,
                                        beta, out, widx, ridx, s),
                s);
}

}  // extern "C"

namespace {

// Shapes the planned scan supports; also bounds its grids (the plan pass
// launches ceil(T/32) 256-thread workgroups per memory).
int check_plan_shape(int B, int H, int64_t N, int d_v, int64_t T) {
  if (B < 1 || H < 1) return fail(SDM_ERR_INVALID, "B and H must be >= 1");
  if ((int64_t)B * H > sdm::kMaxMemories)
    return fail(SDM_ERR_UNSUPPORTED, "B*H must be at most 2^20 memories per call");
  if (T < 0) return fail(SDM_ERR_INVALID, "T must be >= 0");
  if (T > sdm::kMaxSteps || (int64_t)B * H * T > sdm::kMaxMemorySteps)
    return fail(SDM_ERR_UNSUPPORTED, "T must be at most 2^32 and B*H*T at most 2^40 per call");
  if ((int64_t)B * H * ((T + sdm::kPlanSteps - 1) / sdm::kPlanSteps) > sdm::kMaxStrideBlocks)
    return fail(SDM_ERR_UNSUPPORTED, "B*H*ceil(T/32) must be below 2^24; split the sequence");
  // a workgroup's slices of the lists and of v are addressed by 32-bit
  // buffer offsets: T * 512 and T * d_v * 4 bytes stay below 2^31
  if (T > sdm::kPlanMaxSteps)
    return fail(SDM_ERR_UNSUPPORTED, "the planned scan takes at most 2^20 steps per call; split the sequence");
  if (N < 1 || N >= ((int64_t)1 << 31))
    return fail(SDM_ERR_INVALID, "N must be in [1, 2^31) (got %lld)", (long long)N);
  if (d_v != 32 && d_v != 64 && d_v != 128 && d_v != 256)
    return fail(SDM_ERR_UNSUPPORTED, "the planned scan needs d_v in {32, 64, 128, 256} (got %d)", d_v);
  if (N * d_v * 4 >= ((int64_t)1 << 31))
    return fail(SDM_ERR_UNSUPPORTED, "one memory's table must be below 2 GiB");
  if (!sdm::ranges::scan_tiles_ok(N, d_v, 4, T, 1, 1, 32, false))
    return fail(SDM_ERR_UNSUPPORTED, "a state tile's buffer range does not fit 31 bits");
  return SDM_OK;
}

int check_workspace(const void* ws, size_t bytes, int B, int H, int d_v, int64_t T) {
  const int S = sdm::planned_shards(B * H, d_v);
  const int64_t need = sdm::plan_layout((int64_t)B * H, S, T, d_v).total;
  if (!ws) return fail(SDM_ERR_INVALID, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(SDM_ERR_INVALID, "workspace must be 256-byte aligned");
  if ((int64_t)bytes < need)
    return fail(SDM_ERR_INVALID, "workspace has %zu bytes, %lld needed", bytes, (long long)need);
  return SDM_OK;
}

}  // namespace

extern "C" {

size_t sdm_scan_plan_workspace_size(int B, int H, int d_v, int64_t T) {
  if (B < 1 || H < 1 || T < 0 || (int64_t)B * H > sdm::kMaxMemories || T > sdm::kPlanMaxSteps)
    return 0;
  if (d_v != 32 && d_v != 64 && d_v != 128 && d_v != 256) return 0;
  const int S = sdm::planned_shards(B * H, d_v);
  return (size_t)sdm::plan_layout((int64_t)B * H, S, T, d_v).total;
}

int sdm_scan_plan(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                  const int32_t* widx, const float* wk, const int32_t* ridx, const float* rw,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_plan_shape(B, H, N, d_v, T))) return rc;
  if (W < 1 || R < 1) return fail(SDM_ERR_INVALID, "W and R must be >= 1");
  if (W > 64 || R > 64) return fail(SDM_ERR_UNSUPPORTED, "W and R above 64 are not compiled");
  if (T == 0) return SDM_OK;
  if (!widx || !wk || !ridx || !rw) return fail(SDM_ERR_INVALID, "an index or weight pointer is NULL");
  if (!aligned(widx, 4) || !aligned(wk, 4) || !aligned(ridx, 4) || !aligned(rw, 4))
    return fail(SDM_ERR_INVALID, "index and weight arrays must be 4-byte aligned");
  if ((rc = check_workspace(workspace, workspace_bytes, B, H, d_v, T))) return rc;
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_scan_plan",
                sdm::launch_scan_plan(B, H, N, d_v, T, W, R, widx, wk, ridx, rw, workspace, s), s);
}

int sdm_scan_planned(void* M, int B, int H, int64_t N, int d_v, int64_t T, const float* v,
                     const float* alpha, const float* beta, float* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_plan_shape(B, H, N, d_v, T))) return rc;
  if (!M) return fail(SDM_ERR_INVALID, "M is NULL");
  if (!aligned(M, 16)) return fail(SDM_ERR_INVALID, "M must be 16-byte aligned");
  if (T == 0) return SDM_OK;
  if (!v || !alpha || !beta || !out) return fail(SDM_ERR_INVALID, "v, alpha, beta and out must not be NULL");
  if (!aligned(v, 4) || !aligned(alpha, 4) || !aligned(beta, 4) || !aligned(out, 16))
    return fail(SDM_ERR_INVALID, "v, alpha, beta must be 4-byte and out 16-byte aligned");
  if ((rc = check_workspace(workspace, workspace_bytes, B, H, d_v, T))) return rc;
  hipStream_t s = (hipStream_t)stream;
  return finish("sdm_scan_planned",
                sdm::launch_scan_planned(reinterpret_cast<float*>(M), B, H, N, d_v, T, v, alpha,
                                         beta, out, workspace, s),
                s);
}

}  // extern "C"
