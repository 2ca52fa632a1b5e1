// Drives the C-ABI layer of libsdm (csrc/api.hip, compiled host-only) under
// AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers
// replaced by stubs that record their arguments and the two HIP runtime calls
// the layer makes replaced by stubs whose results the driver sets.  Checks:
// valid calls reach their launcher with the caller's sizes; invalid calls are
// rejected with the right status and a message before any launcher runs;
// launch and (with SDM_DEBUG_SYNC=1) kernel errors map to SDM_ERR_HIP; the
// error text is per thread; extreme sizes are rejected without overflow.
// Prints "ok" and exits 0 when every check passes.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>

#include "../../include/sdm.h"

namespace {
int g_launches = 0;               // launcher calls so far
hipError_t g_launch_rc = hipSuccess;
hipError_t g_sync_rc = hipSuccess;
int g_syncs = 0;
long long g_last[8];              // sizes the last launcher received
int g_fails = 0;

void check(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAIL line %d: %s (last error: %s)\n", line, what, sdm_last_error());
    ++g_fails;
  }
}
#define CHECK(x) check((x), #x, __LINE__)

hipError_t record(long long a = 0, long long b = 0, long long c = 0, long long d = 0,
                  long long e = 0, long long f = 0, long long g = 0, long long h = 0) {
  ++g_launches;
  const long long v[8] = {a, b, c, d, e, f, g, h};
  std::memcpy(g_last, v, sizeof v);
  return g_launch_rc;
}
}  // namespace

extern "C" {
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }
hipError_t hipStreamSynchronize(hipStream_t) {
  ++g_syncs;
  return g_sync_rc;
}
}

namespace sdm {
hipError_t launch_project(const uint16_t*, const uint16_t*, int B, int T, int d_model, int H,
                          int n, int d_v, float*, float*, float*, float*, float*, float*, float*,
                          hipStream_t) {
  return record(B, T, d_model, H, n, d_v);
}
hipError_t launch_select(const float*, const float*, int64_t units, int n, int K, int32_t*,
                         float*, float*, hipStream_t) {
  return record(units, n, K);
}
hipError_t launch_state_init(void*, int dtype, const float*, int B, int H, int64_t N, int d_v,
                             hipStream_t) {
  return record(dtype, B, H, N, d_v);
}
hipError_t launch_scan(void*, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W,
                       int R, const int32_t*, const float*, const int32_t*, const float*,
                       const float*, const float*, const float*, float*, void* tape,
                       hipStream_t) {
  return record(dtype, B, H, N, d_v, T, W * 1000 + R, tape != nullptr);
}
hipError_t launch_step_decode(void*, int dtype, int B, int H, int n, int d_v, int W, int R,
                              const float*, const float*, const float*, const float*,
                              const float*, const float*, const float*, float*, int32_t*,
                              int32_t*, hipStream_t) {
  return record(dtype, B, H, n, d_v, W, R);
}
size_t scan_backward_workspace_bytes(int n_mem, int d_v, int64_t T, int W, int R) {
  return (size_t)n_mem * (size_t)T * (size_t)(d_v / 16) * (size_t)(W + R + 1) * 4;
}
hipError_t launch_scan_backward(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                                const int32_t*, const float*, const int32_t*, const float*,
                                const float*, const float*, const float*, const float*,
                                const float*, float*, float*, float*, float*, float*, float*,
                                const uint64_t* first, float*, hipStream_t) {
  return record(B, H, N, d_v, T, W, R, first != nullptr);
}
hipError_t static_scratch(void** ptr) {
  static float fake[4] __attribute__((aligned(256)));
  *ptr = fake;
  return hipSuccess;
}
hipError_t launch_select_backward(const int32_t*, const float*, const float*, int64_t units,
                                  int n, int K, float*, float*, hipStream_t) {
  return record(units, n, K);
}
hipError_t launch_state_init_backward(const float*, int B, int H, int64_t N, int d_v,
                                      const uint32_t* seen, float*, hipStream_t) {
  return record(B, H, N, d_v, seen != nullptr);
}
hipError_t launch_touch_prepare(int B, int H, int64_t N, int64_t T, int W, int R,
                                const int32_t*, const int32_t*, uint32_t*, uint64_t*,
                                hipStream_t) {
  return record(B, H, N, T, W, R);
}
int planned_shards(int n_mem, int d_v) {  // as the library's rule on 256 compute units
  const int64_t units = (int64_t)n_mem * (d_v / 32);
  if (units * 2 > 256) return 1;
  if (units * 4 > 256) return 2;
  return 8;
}
hipError_t launch_scan_plan(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                            const int32_t*, const float*, const int32_t*, const float*, void*,
                            hipStream_t) {
  return record(B, H, N, d_v, T, W, R, 1);
}
hipError_t launch_scan_planned(float*, int B, int H, int64_t N, int d_v, int64_t T, const float*,
                               const float*, const float*, float*, void*, hipStream_t) {
  return record(B, H, N, d_v, T, 0, 0, 2);
}
}  // namespace sdm

int main() {
  setenv("SDM_DEBUG_SYNC", "1", 1);  // read once, at the first call
  // Non-null, 16-byte aligned addresses that are never dereferenced.
  static float buf[64] __attribute__((aligned(16)));
  float* F = buf;
  int32_t* I = reinterpret_cast<int32_t*>(buf);
  uint64_t* U = reinterpret_cast<uint64_t*>(buf);
  void* V = buf;
  const int64_t big = (int64_t)1 << 62;

  // ---- sdm_select
  int n0 = g_launches;
  CHECK(sdm_select(F, F, 1000, 1024, 64, I, F, F, nullptr) == SDM_OK);
  CHECK(g_launches == n0 + 1 && g_last[0] == 1000 && g_last[1] == 1024 && g_last[2] == 64);
  CHECK(g_syncs == 1);  // SDM_DEBUG_SYNC=1 waits after every call
  n0 = g_launches;
  CHECK(sdm_select(nullptr, F, 10, 64, 8, I, F, F, nullptr) == SDM_ERR_INVALID);
  CHECK(std::strstr(sdm_last_error(), "x1") != nullptr);
  CHECK(sdm_select(F, F, -1, 64, 8, I, F, F, nullptr) == SDM_ERR_INVALID);
  CHECK(sdm_select(F, F, big, 64, 8, I, F, F, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_select(F, F, 10, 100, 8, I, F, F, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_select(F, F, 10, 64, 0, I, F, F, nullptr) == SDM_ERR_INVALID);
  CHECK(sdm_select(F, F, 10, 1 << 30, 8, I, F, F, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_select(F + 1, F, 10, 256, 8, I, F, F, nullptr) == SDM_ERR_INVALID);
  CHECK(g_launches == n0);
  CHECK(sdm_select(nullptr, nullptr, 0, 64, 8, nullptr, nullptr, nullptr, nullptr) == SDM_OK);
  CHECK(g_launches == n0);  // units = 0: nothing to launch

  // ---- sdm_project
  const uint16_t* X = reinterpret_cast<const uint16_t*>(buf);
  n0 = g_launches;
  CHECK(sdm_project(X, X, 8, 4096, 4096, 8, 1024, 128, F, F, F, F, F, F, F, nullptr) == SDM_OK);
  CHECK(g_launches == n0 + 1 && g_last[0] == 8 && g_last[1] == 4096 && g_last[2] == 4096 &&
        g_last[3] == 8 && g_last[4] == 1024 && g_last[5] == 128);
  n0 = g_launches;
  CHECK(sdm_project(X, X, 1, 10, 96, 1, 4, 4, F, F, F, F, F, F, F, nullptr) ==
        SDM_ERR_UNSUPPORTED);
  CHECK(std::strstr(sdm_last_error(), "multiple of 64") != nullptr);
  CHECK(sdm_project(X, X, 1, 10, 64, 1 << 20, 1 << 20, 4, F, F, F, F, F, F, F, nullptr) ==
        SDM_ERR_UNSUPPORTED);  // H*P beyond 2^31
  CHECK(sdm_project(X, X, 1 << 30, 1 << 30, 64, 1, 4, 4, F, F, F, F, F, F, F, nullptr) ==
        SDM_ERR_UNSUPPORTED);  // too many tiles
  CHECK(sdm_project(X, X, 1, 10, 64, 1, 4, 4, F, F, F, nullptr, F, F, F, nullptr) ==
        SDM_ERR_INVALID);
  CHECK(std::strstr(sdm_last_error(), "q2") != nullptr);
  CHECK(sdm_project(X + 1, X, 1, 10, 64, 1, 4, 4, F, F, F, F, F, F, F, nullptr) ==
        SDM_ERR_INVALID);
  CHECK(sdm_project(X, X, -1, 10, 64, 1, 4, 4, F, F, F, F, F, F, F, nullptr) == SDM_ERR_INVALID);
  CHECK(sdm_project(X, X, 1, 10, 64, 1, 0, 4, F, F, F, F, F, F, F, nullptr) == SDM_ERR_INVALID);
  CHECK(g_launches == n0);
  CHECK(sdm_project(nullptr, nullptr, 0, 10, 64, 1, 4, 4, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr) == SDM_OK);
  CHECK(g_launches == n0);  // no tokens: nothing to launch

  // ---- launch and kernel errors
  g_launch_rc = hipErrorInvalidValue;
  CHECK(sdm_select(F, F, 10, 64, 8, I, F, F, nullptr) == SDM_ERR_HIP);
  CHECK(std::strstr(sdm_last_error(), "launch failed: stub error") != nullptr);
  g_launch_rc = hipSuccess;
  g_sync_rc = hipErrorIllegalAddress;
  CHECK(sdm_state_init(V, SDM_F32, F, 2, 3, 4096, 16, nullptr) == SDM_ERR_HIP);
  CHECK(std::strstr(sdm_last_error(), "kernel failed") != nullptr);
  g_sync_rc = hipSuccess;
  CHECK(sdm_state_init(V, SDM_BF16, F, 2, 3, 4096, 16, nullptr) == SDM_OK);
  CHECK(sdm_last_error()[0] == '\0');  // cleared by a successful call
  CHECK(g_last[0] == SDM_BF16 && g_last[1] == 2 && g_last[2] == 3 && g_last[3] == 4096);

  // ---- per-thread error text
  CHECK(sdm_state_init(nullptr, SDM_F32, F, 1, 1, 16, 16, nullptr) == SDM_ERR_INVALID);
  std::string other;
  std::thread th([&] { other = sdm_last_error(); });
  th.join();
  CHECK(other.empty() && sdm_last_error()[0] != '\0');

  // ---- sdm_state_init
  n0 = g_launches;
  CHECK(sdm_state_init(V, 7, F, 1, 1, 16, 16, nullptr) == SDM_ERR_INVALID);
  CHECK(sdm_state_init(V, SDM_F32, F, 1, 1, big, 16, nullptr) == SDM_ERR_INVALID);
  CHECK(sdm_state_init(V, SDM_FP8, F, 1, 1, 16, 16, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_state_init(V, SDM_F32, F, 0, 1, 16, 16, nullptr) == SDM_ERR_INVALID);
  CHECK(g_launches == n0);

  // ---- sdm_scan / sdm_scan_train
  n0 = g_launches;
  CHECK(sdm_scan(V, SDM_F32, 8, 8, 1 << 20, 128, 4096, 64, 64, I, F, I, F, F, F, F, F,
                 nullptr) == SDM_OK);
  CHECK(g_launches == n0 + 1 && g_last[3] == (1 << 20) && g_last[5] == 4096 &&
        g_last[6] == 64064 && g_last[7] == 0);
  CHECK(sdm_scan_train(V, 2, 2, 4096, 64, 100, 32, 16, I, F, I, F, F, F, F, F, F, nullptr) ==
        SDM_OK);
  CHECK(g_last[7] == 1);
  n0 = g_launches;
  CHECK(sdm_scan(V, SDM_F32, 1, 1, 4096, 16, big, 8, 8, I, F, I, F, F, F, F, F, nullptr) ==
        SDM_ERR_UNSUPPORTED);
  CHECK(sdm_scan_train(V, 1, 1, 4096, 16, big, 8, 8, I, F, I, F, F, F, F, F, F, nullptr) ==
        SDM_ERR_UNSUPPORTED);
  CHECK(sdm_scan(V, SDM_F32, 1 << 30, 1 << 30, 4096, 16, 8, 8, 8, I, F, I, F, F, F, F, F,
                 nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_scan(V, SDM_F32, 1, 1, (int64_t)1 << 30, 256, 8, 8, 8, I, F, I, F, F, F, F, F,
                 nullptr) == SDM_ERR_UNSUPPORTED);  // 1 TiB table
  CHECK(sdm_scan(V, SDM_F32, 1, 1, 4096, 16, 8, 8, 8, nullptr, F, I, F, F, F, F, F, nullptr) ==
        SDM_ERR_INVALID);
  CHECK(sdm_scan(V, SDM_F32, 1, 1, 4096, 16, 8, 8, 8, I, F, I, F, F + 1, F, F, F, nullptr) ==
        SDM_ERR_INVALID);
  CHECK(g_launches == n0);

  // ---- sdm_step_decode
  n0 = g_launches;
  CHECK(sdm_step_decode(V, SDM_BF16, 64, 4, 1024, 128, 64, 64, F, F, F, F, F, F, F, F, I, I,
                        nullptr) == SDM_OK);
  CHECK(g_launches == n0 + 1 && g_last[3] == 1024 && g_last[5] == 64);
  CHECK(sdm_step_decode(V, SDM_FP8, 64, 4, 1024, 128, 64, 64, F, F, F, F, F, F, F, F, I, I,
                        nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_step_decode(V, SDM_F32, 1 << 30, 1 << 30, 64, 128, 8, 8, F, F, F, F, F, F, F, F,
                        nullptr, nullptr, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(g_launches == n0 + 1);

  // ---- sdm_scan_backward and its workspace
  const size_t ws = sdm_scan_backward_workspace_size(2, 2, 64, 100, 32, 16);
  CHECK(ws == (size_t)4 * 100 * 4 * 49 * 4);
  CHECK(sdm_scan_backward_workspace_size(1, 1, 48, 10, 8, 8) == 0);
  n0 = g_launches;
  CHECK(sdm_scan_backward(2, 2, 4096, 64, 100, 32, 16, I, F, I, F, F, F, F, F, F, F, F, F, F,
                          F, F, U, V, ws, nullptr) == SDM_OK);
  CHECK(g_launches == n0 + 1 && g_last[4] == 100 && g_last[7] == 1);
  CHECK(sdm_scan_backward(2, 2, 4096, 64, 100, 32, 16, I, F, I, F, F, F, F, F, F, F, F, F, F,
                          F, F, U, V, ws - 4, nullptr) == SDM_ERR_INVALID);
  CHECK(sdm_scan_backward(1, 1, 4096, 16, big, 8, 8, I, F, I, F, F, F, F, F, F, F, F, F, F, F,
                          F, nullptr, V, (size_t)-1, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_scan_backward(1 << 8, 1 << 8, 4096, 16, 1 << 10, 8, 8, I, F, I, F, F, F, F, F, F,
                          F, F, F, F, F, F, nullptr, V, (size_t)-1, nullptr) ==
        SDM_ERR_UNSUPPORTED);
  CHECK(g_launches == n0 + 1);
  // the allocation-free variant: same checks, its 64 MiB static workspace bound
  n0 = g_launches;
  CHECK(sdm_scan_backward_noalloc(2, 2, 4096, 64, 100, 32, 16, I, F, I, F, F, F, F, F, F, F, F,
                                  F, F, F, F, U, nullptr) == SDM_OK);
  CHECK(g_launches == n0 + 1 && g_last[4] == 100 && g_last[7] == 1);
  // 64 memories x 4096 steps x 8 tiles x 129 sums x 4 bytes = 1.08 GB: too large
  CHECK(sdm_scan_backward_noalloc(8, 8, 4096, 128, 4096, 64, 64, I, F, I, F, F, F, F, F, F, F,
                                  F, F, F, F, F, nullptr, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(std::strstr(sdm_last_error(), "static buffer") != nullptr);
  CHECK(sdm_scan_backward_noalloc(1, 1, 4096, 16, 8, 8, 8, I, F, I, F, F, F, F, F, nullptr, F,
                                  F, F, F, F, F, nullptr, nullptr) == SDM_ERR_INVALID);
  CHECK(g_launches == n0 + 1);

  // ---- selection gradient, M0 gradient, bookkeeping
  n0 = g_launches;
  CHECK(sdm_select_backward(I, F, F, 500, 256, 32, F, F, nullptr) == SDM_OK);
  CHECK(sdm_select_backward(I, F, F, big, 256, 32, F, F, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_state_init_backward(F, 3, 2, 4096, 16, nullptr, F, nullptr) == SDM_OK);
  CHECK(g_last[4] == 0);
  CHECK(sdm_state_init_backward(F, 3, 2, 4096, 16, reinterpret_cast<uint32_t*>(buf) , F,
                                nullptr) == SDM_OK);
  CHECK(g_last[4] == 1);
  CHECK(sdm_touch_prepare(2, 3, 4096, 50, 8, 8, I, I, reinterpret_cast<uint32_t*>(buf), U,
                          nullptr) == SDM_OK);
  CHECK(g_last[3] == 50);
  CHECK(sdm_touch_prepare(2, 3, 4096, big, 8, 8, I, I, reinterpret_cast<uint32_t*>(buf), U,
                          nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(sdm_touch_prepare(1 << 30, 1 << 30, 4096, 50, 8, 8, I, I,
                          reinterpret_cast<uint32_t*>(buf), U, nullptr) == SDM_ERR_UNSUPPORTED);
  CHECK(g_launches == n0 + 4);

  // ---- planned scan
  {
    static float ws_buf[64] __attribute__((aligned(256)));
    void* WS = ws_buf;
    const size_t need = sdm_scan_plan_workspace_size(1, 16, 128, 16384);
    // 16 memories x 8 shards x 16384 steps of lists, plus 8 partial outputs
    const size_t lists = (size_t)16 * 8 * 16384 * (4 + 512 + 512 + 128 + 128);
    CHECK(need == lists + (size_t)8 * 16 * 16384 * 128 * 4);
    CHECK(sdm_scan_plan_workspace_size(1, 16, 16, 100) == 0);
    CHECK(sdm_scan_plan_workspace_size(0, 16, 128, 100) == 0);
    CHECK(sdm_scan_plan_workspace_size(1, 16, 128, -1) == 0);
    CHECK(sdm_scan_plan_workspace_size(1 << 30, 1 << 30, 128, 100) == 0);
    CHECK(sdm_scan_plan_workspace_size(64, 4, 128, 100) ==
          (size_t)256 * 100 * (4 + 512 + 512 + 128 + 128));  // S = 1: no partials
    n0 = g_launches;
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 128, 16384, 64, 64, I, F, I, F, WS, need, nullptr) ==
          SDM_OK);
    CHECK(g_launches == n0 + 1 && g_last[1] == 16 && g_last[2] == (1 << 20) && g_last[4] == 16384 &&
          g_last[7] == 1);
    CHECK(sdm_scan_planned(V, 1, 16, 1 << 20, 128, 16384, F, F, F, F, WS, need, nullptr) == SDM_OK);
    CHECK(g_launches == n0 + 2 && g_last[3] == 128 && g_last[7] == 2);
    n0 = g_launches;
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 128, 16384, 64, 64, I, F, I, F, WS, need - 1, nullptr) ==
          SDM_ERR_INVALID);
    CHECK(std::strstr(sdm_last_error(), "needed") != nullptr);
    CHECK(sdm_scan_planned(V, 1, 16, 1 << 20, 128, 16384, F, F, F, F, WS, need - 1, nullptr) ==
          SDM_ERR_INVALID);
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 128, 100, 64, 64, I, F, I, F, F + 1, need, nullptr) ==
          SDM_ERR_INVALID);  // workspace not 256-byte aligned
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 16, 100, 64, 64, I, F, I, F, WS, need, nullptr) ==
          SDM_ERR_UNSUPPORTED);  // d_v 16
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 128, 100, 65, 64, I, F, I, F, WS, need, nullptr) ==
          SDM_ERR_UNSUPPORTED);
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 128, 100, 64, 64, nullptr, F, I, F, WS, need, nullptr) ==
          SDM_ERR_INVALID);
    CHECK(sdm_scan_plan(1, 16, (int64_t)1 << 31, 128, 100, 64, 64, I, F, I, F, WS, need,
                        nullptr) == SDM_ERR_INVALID);
    CHECK(sdm_scan_plan(1, 16, 1 << 23, 128, 100, 64, 64, I, F, I, F, WS, need, nullptr) ==
          SDM_ERR_UNSUPPORTED);  // 4 GiB table
    CHECK(sdm_scan_plan(1 << 20, 1, 1 << 10, 32, (int64_t)1 << 20, 8, 8, I, F, I, F, WS, need,
                        nullptr) == SDM_ERR_UNSUPPORTED);  // plan grid beyond 2^24 blocks
    // at most 2^20 steps per call (the workgroups' list slices are addressed by 31-bit offsets)
    CHECK(sdm_scan_plan_workspace_size(1, 16, 128, ((int64_t)1 << 20) + 1) == 0);
    CHECK(sdm_scan_plan_workspace_size(1, 16, 128, (int64_t)1 << 20) > 0);
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 128, ((int64_t)1 << 20) + 1, 64, 64, I, F, I, F, WS, need,
                        nullptr) == SDM_ERR_UNSUPPORTED);
    CHECK(std::strstr(sdm_last_error(), "2^20 steps") != nullptr);
    CHECK(sdm_scan_planned(V, 1, 16, 1 << 20, 128, ((int64_t)1 << 20) + 1, F, F, F, F, WS, need,
                           nullptr) == SDM_ERR_UNSUPPORTED);
    CHECK(std::strstr(sdm_last_error(), "2^20 steps") != nullptr);
    CHECK(sdm_scan_planned(nullptr, 1, 16, 1 << 20, 128, 100, F, F, F, F, WS, need, nullptr) ==
          SDM_ERR_INVALID);
    CHECK(sdm_scan_planned(V, 1, 16, 1 << 20, 128, 100, F, F, F, F + 1, WS, need, nullptr) ==
          SDM_ERR_INVALID);  // out not 16-byte aligned
    CHECK(g_launches == n0);
    CHECK(sdm_scan_plan(1, 16, 1 << 20, 128, 0, 64, 64, nullptr, nullptr, nullptr, nullptr,
                        nullptr, 0, nullptr) == SDM_OK);
    CHECK(sdm_scan_planned(V, 1, 16, 1 << 20, 128, 0, nullptr, nullptr, nullptr, nullptr, nullptr,
                           0, nullptr) == SDM_OK);
    CHECK(g_launches == n0);  // T = 0: nothing to launch
  }

  CHECK(std::strcmp(sdm_status_string(SDM_ERR_HIP), "SDM_ERR_HIP") == 0);
  CHECK(std::strcmp(sdm_status_string(42), "unknown status") == 0);
  if (g_fails) return 1;
  std::printf("ok\n");
  return 0;
}
