// Kernel instantiations for dtype f32, op avg.
#define AR_LAUNCH_DEFINITIONS
#include "launch.h"

namespace ar {
AR_INSTANTIATE_LAUNCHES(1, 2)
}  // namespace ar
