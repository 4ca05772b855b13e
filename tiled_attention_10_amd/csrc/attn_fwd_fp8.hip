// FP8 attention forward: not built yet.
#include "tattn_launch.hpp"

namespace tattn {
hipError_t launch_attn_fwd_fp8(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace tattn
