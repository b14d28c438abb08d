// moe_phase1_256.hip -- Phase 1 at 256 x 256 tiles (I >= 256, B >= 256).
#include "moe_phase1.hpp"

namespace mx {

template hipError_t phase1_launch<256, 256, false>(Phase1Args, int, int, hipStream_t);

}  // namespace mx
