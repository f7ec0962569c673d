// Stand-ins for the kernel launchers, for the host-only build of the library
// (api.cpp and planner.cpp built with the host compiler's sanitizers). Every
// compute entry point validates its arguments before it reaches a launcher;
// in this build a call that passes validation gets SKV_ERR_HIP instead of a
// kernel.
#include "internal.hpp"

namespace skv {
hipError_t launch_gqa_valu(const AttnLaunch&) { return hipErrorNoDevice; }
hipError_t launch_gqa_mfma(const AttnLaunch&) { return hipErrorNoDevice; }
hipError_t launch_mla_mfma(const AttnLaunch&) { return hipErrorNoDevice; }
hipError_t launch_merge(const MergeLaunch&) { return hipErrorNoDevice; }
hipError_t launch_hbm_probe(const void*, int64_t, uint32_t*, int, hipStream_t) { return hipErrorNoDevice; }
}  // namespace skv
