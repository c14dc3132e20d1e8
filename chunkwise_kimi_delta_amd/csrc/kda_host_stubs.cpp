// Host-only stand-ins for the kernel launchers, linked into the sanitizer
// build of the C ABI (kda_api.cpp) so that its validation, workspace planning
// and error paths run under AddressSanitizer and UndefinedBehaviorSanitizer
// on a machine without a GPU.  They launch nothing and report success.
#include <cstdio>

#include "kda_bwd_launch.h"

namespace kda {
hipError_t launch_chunk_offsets(const int32_t*, int, int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_intra(int, int, int, const IntraArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_scan(int, int, int, const ScanArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_merge(int, int, const MergeArgs&, hipStream_t, bool) { return hipSuccess; }
hipError_t launch_prefix_merge(int, int, const PrefixMergeArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_recurrent(int, int, int, const RecurrentArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd(int, int, int, const BwdArgs&, int, int64_t, float*, hipStream_t) { return hipSuccess; }
// (no device scratch in a host-only build)
hipError_t noalloc_scratch(hipStream_t, void**, char* why, size_t why_len) {
  snprintf(why, why_len, "host-only build");
  return hipErrorNotSupported;
}
}  // namespace kda
