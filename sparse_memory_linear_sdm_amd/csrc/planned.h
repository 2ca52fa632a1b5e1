// Planned scan (scan_planned.hip) behind the C ABI: workspace layout,
// shard count and launchers (host side).  Arguments are validated by the
// C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

// Planned scan (scan_planned.hip), fp32 state in 32-column tiles.  The plan
// pass writes, per (memory, row shard, step), the step's write and read rows
// of that shard compacted into lists, and the scan pass reads only its
// shard's lists.  Workspace layout (byte offsets, each 256-byte aligned):
//   hdr  [n_mem, S, T]      uint32   rows in the write list | read list << 8 |
//                                    forwarded-row flag << 16
//   went [n_mem, S, T, 64]  uint2    (row, weight bits) of the write list
//   rent [n_mem, S, T, 64]  uint2    the same for the read list
//   srcw [n_mem, S, T, 64]  uint16   where a write row's current value lives
//   srcr [n_mem, S, T, 64]  uint16   the same for a read row
//   part [S, n_mem, T, d_v] float    per-shard read sums (S > 1 only)
// A src entry is 0 (the row as gathered is current) or 1 + a*64 + j: the
// value written by step u - a at position j of its write list, a in
// [0, kPlanLookback] (a >= 1 for write rows).  srcw and srcr are written only
// for (memory, shard, step) entries whose flag is set.
constexpr int kPlanLookback = 8;
struct PlanLayout {
  int64_t hdr, went, rent, srcw, srcr, part, total;
};
inline PlanLayout plan_layout(int64_t n_mem, int S, int64_t T, int d_v) {
  auto up = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
  const int64_t units = n_mem * S * T;
  PlanLayout L{};
  int64_t o = 0;
  L.hdr = o;  o = up(o + units * 4);
  L.went = o; o = up(o + units * 64 * 8);
  L.rent = o; o = up(o + units * 64 * 8);
  L.srcw = o; o = up(o + units * 64 * 2);
  L.srcr = o; o = up(o + units * 64 * 2);
  L.part = o; o = up(o + (S > 1 ? (int64_t)S * n_mem * T * d_v * 4 : 0));
  L.total = o;
  return L;
}
// Row shards per (memory, tile) the planned scan uses: 1, 2 or 8.
int planned_shards(int n_mem, int d_v);
// Steps per plan workgroup.
constexpr int kPlanSteps = 32;
// Steps per planned call (32-bit offsets into a workgroup's slices).
constexpr int64_t kPlanMaxSteps = (int64_t)1 << 20;
hipError_t launch_scan_plan(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                            const int32_t* widx, const float* wk, const int32_t* ridx,
                            const float* rw, void* ws, hipStream_t stream);
hipError_t launch_scan_planned(float* M, int B, int H, int64_t N, int d_v, int64_t T,
                               const float* v, const float* alpha, const float* beta, float* out,
                               void* ws, hipStream_t stream);

}  // namespace sdm
