// attn_bwd.hip - straight-through backward (work in progress).
#include "aq_device.hpp"
#include "launch.hpp"

namespace aq {
hipError_t launch_attn_bwd(const AttnArgs &, const BwdArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace aq
