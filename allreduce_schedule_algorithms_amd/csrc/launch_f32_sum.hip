// Kernel instantiations for dtype f32, op sum.
#define AR_LAUNCH_DEFINITIONS
#include "launch.h"

namespace ar {
AR_INSTANTIATE_LAUNCHES(1, 0)
}  // namespace ar
