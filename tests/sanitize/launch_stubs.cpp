// Stand-ins for the kernel launchers, for the host-only sanitizer build of the
// C ABI layer: every one reports a launch error, so a call that gets past
// validation shows as WKV7_ERR_LAUNCH and no device code exists to reach.
#include "wkv7_internal.h"

namespace wkv7 {
hipError_t launch_seq_fwd(const FwdArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd(const FwdArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd128(const FwdArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd128_split(const FwdArgs&, const FwdSplit&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd_split(const FwdArgs&, int, const FwdSplit&, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_seq_fwd_split(const FwdArgs&, const FwdSplit&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_seg_combine(int, int, float*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd_sequential(const FwdArgs&, int, int, int, float*, int*, int, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_bwd(const BwdArgs&, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_seq_bwd(const SeqBwdArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_state_copy(int, int, const float*, float*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_epilogue(const EpiArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk_fwd_epilogue(const FwdArgs&, const EpiParams&, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t static_scratch(void** ptr) {
    *ptr = nullptr;
    return hipErrorInvalidValue;
}
}  // namespace wkv7
