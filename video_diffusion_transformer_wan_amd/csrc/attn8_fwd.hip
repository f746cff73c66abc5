// 8-bit attention, stage 2 (placeholder until the kernel lands).
#include "wan_attn_internal.h"

namespace wan {
hipError_t launch_attn8_fwd(const int8_t*, const float*, const int8_t*, const float*, const uint8_t*,
                            const float*, void*, const AttnShape&, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace wan
