// Kernel instantiations for dtype i32, op max.
#define AR_LAUNCH_DEFINITIONS
#include "launch.h"

namespace ar {
AR_INSTANTIATE_LAUNCHES(0, 1)
}  // namespace ar
