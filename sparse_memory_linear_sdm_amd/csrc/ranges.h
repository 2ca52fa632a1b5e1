// Byte ranges of the raw buffer resources ("descriptors") that the scan, the
// training forward, the reverse scan and the bookkeeping kernel build, kept
// in one place: the kernels build their descriptors from these functions,
// the C-ABI layer checks them for the caller's sizes before it launches
// anything, and a host test checks them for every shape the GPU tests use.
// Plain C++ (constexpr functions are callable from HIP device code as well),
// no HIP dependency, so the host test builds it with g++.
//
// How the kernels use a descriptor.  Each one covers a tile of `tile_bytes`
// columns of a row-major table of `rows` rows of `row_bytes` bytes, starting
// at the tile's first column, and its range (the descriptor's record count)
// runs to the end of the table.  A valid access of row r reads or writes
// bytes [r * row_bytes + o, r * row_bytes + o + 16) for a lane offset
// o + 16 <= tile_bytes; an access that is not to happen gets the offset
// kOffNone = 2^31 (plus at most kOffExtra bytes), which must lie past the
// range, so that the hardware returns zero for the load and drops the store.
// So for every tile the kernels may use:
//   0 <= range < 2^31        (a negative range, handed over as a 32-bit record
//                            count, would become ~4 G and switch the check off),
//   last valid end <= range  (the last row's tile fragment lies inside).
#pragma once
#include <stdint.h>

namespace sdm {
namespace ranges {

constexpr uint32_t kOffNone = 0x80000000u;
// Largest amount added to kOffNone by any kernel (a lane's column offset and
// the scan prologue's distinct dummy stores); kOffNone + kOffExtra + 16 must
// not wrap in 32 bits.
constexpr int64_t kOffExtra = 4096;
constexpr int64_t kRangeLimit = (int64_t)1 << 31;

// Range of the descriptor of column tile `tile` (tile * tile_bytes bytes into
// each row) of a [rows, row_bytes] table.
constexpr int64_t table_range(int64_t rows, int64_t row_bytes, int64_t tile,
                              int64_t tile_bytes) {
  return rows * row_bytes - tile * tile_bytes;
}

// End offset of the last valid access through that descriptor: the last
// row's tile fragment.
constexpr int64_t table_end(int64_t rows, int64_t row_bytes, int64_t tile_bytes) {
  return (rows - 1) * row_bytes + tile_bytes;
}

constexpr bool span_ok(int64_t range, int64_t end) {
  return range >= 0 && range < kRangeLimit && end <= range &&
         (int64_t)kOffNone >= range && (int64_t)kOffNone + kOffExtra + 16 <= ((int64_t)1 << 32);
}

// Every tile descriptor of a table split into ntiles tiles of tile_bytes.
constexpr bool tiles_ok(int64_t rows, int64_t row_bytes, int64_t tile_bytes, int64_t ntiles) {
  if (rows < 1 || row_bytes < 1 || tile_bytes < 16 || ntiles < 1 ||
      ntiles * tile_bytes > row_bytes)
    return false;
  for (int64_t t = 0; t < ntiles; ++t)
    if (!span_ok(table_range(rows, row_bytes, t, tile_bytes), table_end(rows, row_bytes, tile_bytes)))
      return false;
  return true;
}

// sdm_scan / sdm_scan_train: the state tile descriptor of every memory and,
// with a tape, the tape tile descriptor ([T * (W + R), d_v] rows per memory),
// for the tile width `cols` the launcher picked (elem_bytes per value).
constexpr bool scan_tiles_ok(int64_t N, int d_v, int elem_bytes, int64_t T, int W, int R, int cols,
                             bool tape) {
  if (T == 0) return true;  // nothing is launched
  const int64_t row_bytes = (int64_t)d_v * elem_bytes, tile_bytes = (int64_t)cols * elem_bytes;
  if (d_v % cols != 0) return false;
  if (!tiles_ok(N, row_bytes, tile_bytes, d_v / cols)) return false;
  return !tape || tiles_ok(T * (W + R), row_bytes, tile_bytes, d_v / cols);
}

// The same for every tile width the scan launcher may pick for this element
// size (16 or 32 columns for fp32 and bf16 state, 32 for fp8).
constexpr bool scan_ok(int64_t N, int d_v, int elem_bytes, int64_t T, int W, int R, bool tape) {
  const int first = elem_bytes == 1 ? 32 : 16;
  for (int cols = first; cols <= 32; cols *= 2)
    if (cols <= d_v && !scan_tiles_ok(N, d_v, elem_bytes, T, W, R, cols, tape)) return false;
  return true;
}

// sdm_scan_backward (fp32): the gradient table G [N, d_v] and the tape
// [T * (W + R), d_v] of every memory, 16- or 32-column tiles.
constexpr bool scan_backward_ok(int64_t N, int d_v, int64_t T, int W, int R) {
  return scan_ok(N, d_v, 4, T, W, R, true);
}

// sdm_touch_prepare: one descriptor per memory over widx [T, W], ridx [T, R]
// (4-byte entries, one per lane) and first [T, 2] (one 16-byte entry per step).
constexpr bool touch_ok(int64_t T, int W, int R) {
  if (T == 0) return true;
  return span_ok(table_range(T * W, 4, 0, 4), table_end(T * W, 4, 4)) &&
         span_ok(table_range(T * R, 4, 0, 4), table_end(T * R, 4, 4)) &&
         span_ok(table_range(T, 16, 0, 16), table_end(T, 16, 16));
}

}  // namespace ranges
}  // namespace sdm
