// Kernel instantiations for dtype bf16, op max.
#define AR_LAUNCH_DEFINITIONS
#include "launch.h"

namespace ar {
AR_INSTANTIATE_LAUNCHES(2, 1)
}  // namespace ar
