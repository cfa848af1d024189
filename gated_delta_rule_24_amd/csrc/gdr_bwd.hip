// Gate-aware backward of the chunkwise forward (placeholder: not built yet).
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

bool bwd_supported(int, int, int, uint32_t) { return false; }

size_t bwd_workspace_bytes(int, int, int, int, int, uint32_t) { return 0; }

hipError_t launch_bwd(const BwdParams&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace gdr
