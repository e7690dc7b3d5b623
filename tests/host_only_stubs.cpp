// Stand-ins for the kernel launchers in a host-only build of the library's
// host sources (tests/sanitize_check.cpp under the host sanitizers).  The
// paths that build exercises never reach the GPU; if one did, it gets an
// error back instead of a launch.
#include "internal.h"

namespace zmi {

hipError_t launch_flatten(const FlatPiece*, int, void*, int*, int, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_scan(const void*, int64_t, int*, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_adam(const void*, float*, float*, float*, uint16_t*, int64_t, int64_t,
                       const int*, const AdamScalars&, const AdamScalars*, int, int, bool,
                       hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_write_param(const float*, uint16_t*, int64_t, int, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_flag_clear(int*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_step_prologue(const int*, const DeviceStep*, AdamScalars*,
                                const zero_adam_hparams_t&, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_step_epilogue(int*, DeviceStep*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_adam_scalars(const zero_adam_hparams_t&, int64_t, int64_t, double, AdamScalars*,
                               hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_offload_snapshot(int*, DeviceStep*, OffloadSlot*, hipStream_t) {
    return hipErrorNoDevice;
}

}  // namespace zmi
