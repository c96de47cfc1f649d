// Backward attention kernels for gfx950 (recomputation from the saved LSE).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

hipError_t launch_bwd(const BwdArgs &, int, bool, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
