// Backward attention kernels for gfx950 (placeholder until the kernels land).
#include "device.h"
#include "kernels.h"

namespace attn {
hipError_t bwd_setup_device() { return hipSuccess; }
hipError_t launch_bwd(const BwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
