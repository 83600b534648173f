// Host-only stand-ins for the kernel launchers of libssscan.so, so that the C ABI's
// argument validation (ss_api.cpp) can be built with the host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU.  Each
// "launch" only reports a status; the validation that precedes it is the real code.
// The status is hipSuccess, or the error code in SS_STUB_LAUNCH_ERROR when that is
// set, so that the library's HIP-failure path can be driven too.
#include <stdlib.h>

#include "ss_internal.h"

namespace {
hipError_t stub_status()
{
    const char* v = getenv("SS_STUB_LAUNCH_ERROR");
    return v ? static_cast<hipError_t>(atoi(v)) : hipSuccess;
}
}  // namespace

namespace ssk {
hipError_t launch_scan(const ScanArgs&, int, hipStream_t) { return stub_status(); }
hipError_t launch_step(const StepArgs&, int, hipStream_t) { return stub_status(); }
hipError_t launch_panel(const ScanArgs&, int, hipStream_t) { return stub_status(); }
hipError_t launch_ckpt_pass(const ScanArgs&, int, hipStream_t) { return stub_status(); }
hipError_t launch_bwd(const BwdArgs&, int, hipStream_t) { return stub_status(); }
hipError_t launch_conv(const ConvArgs&, int, int, hipStream_t) { return stub_status(); }
hipError_t launch_ssd(const SsdArgs&, hipStream_t) { return stub_status(); }
hipError_t scratch_pointer(void** p)
{
    static char buf[256] __attribute__((aligned(256)));
    *p = buf;
    return hipSuccess;
}
}  // namespace ssk
