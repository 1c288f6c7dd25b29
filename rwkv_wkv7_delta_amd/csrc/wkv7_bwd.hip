// wkv7_bwd.hip -- placeholder until the chunked adjoint kernel lands.
#include "wkv7_device.h"
#include "wkv7_internal.h"
namespace wkv7 {
hipError_t launch_bwd(const BwdArgs&, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace wkv7
