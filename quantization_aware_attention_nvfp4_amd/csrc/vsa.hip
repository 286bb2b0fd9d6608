// vsa.hip - cube-sparse forward (work in progress).
#include "aq_device.hpp"
#include "launch.hpp"

namespace aq {
hipError_t launch_vsa_fwd(const AttnArgs &, const VsaArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace aq
