// Host check of the buffer ranges the scan kernels build (ranges.h), compiled
// with g++ alone.  Reads lines "kind N d_v elem_bytes T W R" (kind: scan,
// train, bwd or touch) and prints, per line, 1 when every descriptor the
// kernels would build for those sizes is valid, else 0.
//
// The line "oldmeta steps d_v tile" prints the range that an earlier version
// of the scan's metadata loader gave its per-chunk v descriptor,
// steps * d_v * 4 - tile * 128, as a signed value: for a chunk past the end
// of the sequence (steps = 0) and a column tile > 0 it is negative, which as
// a 32-bit record count switches the range check off.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../sparse_memory_linear_sdm_amd/csrc/ranges.h"

using namespace sdm::ranges;

int main() {
  char kind[16];
  long long a, b, c, d, e, f;
  while (std::scanf("%15s", kind) == 1) {
    if (!std::strcmp(kind, "oldmeta")) {
      if (std::scanf("%lld %lld %lld", &a, &b, &c) != 3) return 2;
      const int64_t range = a * b * 4 - c * 32 * 4;
      std::printf("%lld %u\n", (long long)range, (unsigned)(int)range);
      continue;
    }
    if (std::scanf("%lld %lld %lld %lld %lld %lld", &a, &b, &c, &d, &e, &f) != 6) return 2;
    bool ok = false;
    if (!std::strcmp(kind, "scan")) ok = scan_ok(a, (int)b, (int)c, d, (int)e, (int)f, false);
    else if (!std::strcmp(kind, "train")) ok = scan_ok(a, (int)b, 4, d, (int)e, (int)f, true);
    else if (!std::strcmp(kind, "bwd")) ok = scan_backward_ok(a, (int)b, d, (int)e, (int)f);
    else if (!std::strcmp(kind, "touch")) ok = touch_ok(d, (int)e, (int)f);
    else return 2;
    std::printf("%d\n", ok ? 1 : 0);
  }
  return 0;
}
