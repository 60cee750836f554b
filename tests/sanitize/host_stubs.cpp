// Stand-ins for the kernel launchers, so the C ABI's host code can be built
// alone under AddressSanitizer and UndefinedBehaviorSanitizer (host code
// only) and driven without a GPU.  The host harness only reaches argument
// checks and size queries; a launch reaching a stub is a test failure.
#include <cstdio>
#include <cstdlib>

#include "../../vocab_wide_logit_amd/csrc/vwl_internal.hpp"

namespace vwl {

[[noreturn]] static void reached(const char *what) {
    std::fprintf(stderr, "host harness reached a launch: %s\n", what);
    std::abort();
}

template <int DS>
hipError_t launch_asym_ds(int, int, const Plan &, const AsymParams &, hipStream_t, hipEvent_t) {
    reached("launch_asym_ds");
}
template hipError_t launch_asym_ds<0>(int, int, const Plan &, const AsymParams &, hipStream_t, hipEvent_t);
template hipError_t launch_asym_ds<1>(int, int, const Plan &, const AsymParams &, hipStream_t, hipEvent_t);
template hipError_t launch_asym_ds<2>(int, int, const Plan &, const AsymParams &, hipStream_t, hipEvent_t);

template <int DS>
int asym_blocks_per_cu_ds(int, int, int) {
    return 0;
}
template int asym_blocks_per_cu_ds<0>(int, int, int);
template int asym_blocks_per_cu_ds<1>(int, int, int);
template int asym_blocks_per_cu_ds<2>(int, int, int);
template int asym_blocks_per_cu_ds<3>(int, int, int);

hipError_t launch_e2sci(int, const Plan &, const AsymParams &, hipStream_t, hipEvent_t) { reached("launch_e2sci"); }
hipError_t launch_xfam(int, const Plan &, const AsymParams &, hipStream_t, hipEvent_t) { reached("launch_xfam"); }
hipError_t launch_rapid(int, const Plan &, const RapidParams &, hipStream_t, hipEvent_t) { reached("launch_rapid"); }
hipError_t launch_lmhead(const LmheadParams &, hipStream_t, hipEvent_t) { reached("launch_lmhead"); }
hipError_t launch_fill_zero(void *, size_t, hipStream_t) { reached("launch_fill_zero"); }
int rapid_blocks_per_cu(int, int) { return 0; }
int lmhead_blocks_per_cu(int) { return 0; }

} // namespace vwl
