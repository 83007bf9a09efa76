// Kernel instantiations for dtype bf16, op sum.
#define AR_LAUNCH_DEFINITIONS
#include "launch.h"

namespace ar {
AR_INSTANTIATE_LAUNCHES(2, 0)
}  // namespace ar
