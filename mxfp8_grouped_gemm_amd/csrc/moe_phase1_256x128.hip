// moe_phase1_256x128.hip -- Phase 1 at 256 x 128 tiles (I >= 256, B = 128).
#include "moe_phase1.hpp"

namespace mx {

template hipError_t phase1_launch<256, 128, false>(Phase1Args, int, int, hipStream_t);

}  // namespace mx
