// Host-only stand-ins for the kernel launchers of libssscan.so, so that the C ABI's
// argument validation (ss_api.cpp) can be built with the host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU.  Each
// "launch" only reports success; the validation that precedes it is the real code.
#include "ss_internal.h"

namespace ssk {
hipError_t launch_scan(const ScanArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_step(const StepArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_panel(const ScanArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd(const BwdArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_conv(const ConvArgs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_ssd(const SsdArgs&, hipStream_t) { return hipSuccess; }
hipError_t scratch_pointer(void** p)
{
    static char buf[256] __attribute__((aligned(256)));
    *p = buf;
    return hipSuccess;
}
}  // namespace ssk
