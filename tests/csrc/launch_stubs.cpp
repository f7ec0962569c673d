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
hipError_t launch_fused_setup(uint8_t*, const MergeLaunch&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gqa_valu_fused(const AttnLaunch&, const FusedLaunch&) { return hipErrorNoDevice; }
hipError_t launch_gqa_mfma_fused(const AttnLaunch&, const FusedLaunch&) { return hipErrorNoDevice; }
hipError_t launch_mla_mfma_fused(const AttnLaunch&, const FusedLaunch&) { return hipErrorNoDevice; }
hipError_t launch_hbm_probe(const void*, int64_t, uint32_t*, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_mfma_probe(const void*, int64_t, int, int, int, int, int, uint32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
}  // namespace skv

// The no-allocation entry point lives beside its device array (built with the
// device compiler only): this build answers every call with SKV_ERR_HIP.
extern "C" skv_status skv_decode_attn_noalloc(const skv_attn_desc*, const void*, const void*, const void*,
                                              const int32_t*, const int32_t*, const skv_plan*, const void*,
                                              int32_t, const float*, const float*, void*, int32_t, float*,
                                              void*) {
  return skv::fail(SKV_ERR_HIP, "host-only build: no device scratch array");
}
