// Split-kernel launchers for one codebook per channel group (8-bit codes).
// The kernel itself is in decode_split.h; these instantiations live in their
// own translation unit so that the two variants compile in parallel.
#include "decode_split.h"

namespace loopvq {

hipError_t launch_decode_split_pg(int D, int C, int bits, bool qf32, const DecodeParams& p, int grid,
                                  hipStream_t s) {
#define LVQ_CASE(d, c, b) if (D == d && C == c && bits == b) return launch_split_t<d, c, b, true, false>(p, qf32, grid, s);
  LVQ_CASE(128, 4, 8) LVQ_CASE(128, 8, 8) LVQ_CASE(128, 2, 8)
  LVQ_CASE(64, 2, 8) LVQ_CASE(64, 4, 8) LVQ_CASE(64, 8, 8)
#undef LVQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace loopvq
