// Kernel instantiations for dtype f32, op max.
#define AR_LAUNCH_DEFINITIONS
#include "launch.h"

namespace ar {
AR_INSTANTIATE_LAUNCHES(1, 1)
}  // namespace ar
