#include "device_common.hpp"
#include "internal.hpp"
namespace skv {
hipError_t launch_mla_mfma(const AttnLaunch&) { return hipErrorNotSupported; }
}  // namespace skv
