// Partial-kernel variants for head_dim 256 over the q4_0 cache (two 4-bit codes per byte, one
// f16 scale per 32 elements): one translation unit per head_dim and cache format, so that the
// variants compile in parallel.
#include "partial.h"

namespace skvd {

int launch_partial_256_3(const Plan &p, const LaunchArgs &la, unsigned grid, void *stream,
                          const KernelEvents &ev, bool dbg) {
  return launch_partial_fmt<256, 3>(p, la, grid, stream, ev, dbg);
}

}  // namespace skvd
