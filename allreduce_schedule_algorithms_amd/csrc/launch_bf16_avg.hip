// Kernel instantiations for dtype bf16, op avg.
#define AR_LAUNCH_DEFINITIONS
#include "launch.h"

namespace ar {
AR_INSTANTIATE_LAUNCHES(2, 2)
}  // namespace ar
