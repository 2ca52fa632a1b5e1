// Launchers behind the C ABI (host side).  Arguments are validated by the
// C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

// A kernel dispatch counts its grid in work-items in a 32-bit field, so no
// launch may hold 2^32 or more of them.  The C-ABI layer keeps every call
// within these bounds before it launches anything:
//   one 64-lane wavefront per unit, four per 256-thread block (selection,
//   selection gradient, the reverse scan's finishing pass over memories x
//   steps): at most 2^26 - 4 units, so ceil(units / 4) * 256 < 2^32;
constexpr int64_t kMaxWaveUnits = ((int64_t)1 << 26) - 4;
//   one or a few workgroups per memory and column tile (scan, reverse scan,
//   decode, bookkeeping): at most 2^20 memories, so blocks * threads stays
//   below 2^31 for every tile width and shard count the launchers pick.
constexpr int64_t kMaxMemories = (int64_t)1 << 20;
//   steps per call: at most 2^32, and at most 2^40 memory-steps (B*H*T), so
//   that byte counts such as B*H*T*d_v*4 and T*(W+R)*d_v*4 stay far inside
//   63 bits;
constexpr int64_t kMaxSteps = (int64_t)1 << 32;
constexpr int64_t kMaxMemorySteps = (int64_t)1 << 40;
//   grid-stride kernels (state init) cap their grid at this many blocks of
//   256 threads and loop over the rest.
constexpr int64_t kMaxStrideBlocks = ((int64_t)1 << 24) - 1;

hipError_t launch_select(const float* x1, const float* x2, int64_t units, int n, int K,
                         int32_t* idx, float* score, float* weight, hipStream_t stream);

// Token projections (project.hip): one workgroup per kProjTile x kProjTile
// tile of the [tokens, H*P] output, d_model a multiple of 64.
constexpr int kProjTile = 256;
inline int64_t project_blocks(int64_t M, int64_t Ncols) {
  return ((M + kProjTile - 1) / kProjTile) * ((Ncols + kProjTile - 1) / kProjTile);
}
hipError_t launch_project(const uint16_t* X, const uint16_t* Wt, int B, int T, int d_model, int H,
                          int n, int d_v, float* s1, float* s2, float* q1, float* q2, float* v,
                          float* alpha, float* beta, hipStream_t stream);

hipError_t launch_state_init(void* M, int dtype, const float* M0, int B, int H, int64_t N,
                             int d_v, hipStream_t stream);

hipError_t launch_scan(void* M, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W,
                       int R, const int32_t* widx, const float* wk, const int32_t* ridx,
                       const float* rw, const float* v, const float* alpha, const float* beta,
                       float* out, void* tape, hipStream_t stream);

hipError_t launch_step_decode(void* M, int dtype, int B, int H, int n, int d_v, int W, int R,
                              const float* s1, const float* s2, const float* q1,
                              const float* q2, const float* v, const float* alpha,
                              const float* beta, float* out, int32_t* widx, int32_t* ridx,
                              hipStream_t stream);

size_t scan_backward_workspace_bytes(int n_mem, int d_v, int64_t T, int W, int R);

hipError_t launch_scan_backward(int B, int H, int64_t N, int d_v, int64_t T, int W,
                                int R, const int32_t* widx, const float* wk,
                                const int32_t* ridx, const float* rw, const float* v,
                                const float* alpha, const float* beta, const float* tape,
                                const float* dout, float* G, float* dv, float* dwk, float* drw,
                                float* dalpha, float* dbeta, const uint64_t* first, float* ws,
                                hipStream_t stream);

// The library's per-GPU scratch buffer (scratch.hip), for callers that cannot
// allocate: kStaticScratchBytes of device memory, aligned to 256 bytes, held
// by every GPU the library runs on until the process ends and shared by every
// call on that GPU.  static_scratch() returns its address on the current
// device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void** ptr);

hipError_t launch_select_backward(const int32_t* idx, const float* w, const float* dw,
                                  int64_t units, int n, int K, float* dx1, float* dx2,
                                  hipStream_t stream);

hipError_t launch_state_init_backward(const float* G, int B, int H, int64_t N, int d_v,
                                      const uint32_t* seen, float* dM0, hipStream_t stream);
// The sparse-mode bookkeeping keeps one N-bit table per memory in LDS.
constexpr int64_t kTouchMaxN = (int64_t)1 << 20;
hipError_t launch_touch_prepare(int B, int H, int64_t N, int64_t T, int W, int R,
                                const int32_t* widx, const int32_t* ridx, uint32_t* seen,
                                uint64_t* first, hipStream_t stream);

}  // namespace sdm
