// Stand-ins for the kernel launchers, for the host-only sanitizer build of
// the ABI's argument validation: every call there is refused before a
// launch, so reaching one of these is itself a failure.
#include <cstdio>
#include <cstdlib>

#include "launch.hpp"

namespace linrec {

static hipError_t unexpected(const char* what)
{
    std::fprintf(stderr, "FAIL: %s reached in a validation-only run\n", what);
    std::abort();
}

hipError_t launch_seg_sum(const ScanLaunch&, hipStream_t) { return unexpected("launch_seg_sum"); }
hipError_t launch_seg_fold(const ScanLaunch&, hipStream_t) { return unexpected("launch_seg_fold"); }
hipError_t launch_fwd_intra(const FwdIntraLaunch&, hipStream_t) { return unexpected("launch_fwd_intra"); }
hipError_t launch_bwd_intra(const BwdIntraLaunch&, hipStream_t) { return unexpected("launch_bwd_intra"); }
hipError_t launch_da_finish(const DaFinishLaunch&, hipStream_t) { return unexpected("launch_da_finish"); }
hipError_t launch_delta_fwd(const DeltaFwdLaunch&, hipStream_t) { return unexpected("launch_delta_fwd"); }
hipError_t launch_delta_bwd(const DeltaBwdLaunch&, hipStream_t) { return unexpected("launch_delta_bwd"); }
hipError_t launch_carry_copy(const float*, float*, int64_t, hipStream_t) { return unexpected("launch_carry_copy"); }

}  // namespace linrec
