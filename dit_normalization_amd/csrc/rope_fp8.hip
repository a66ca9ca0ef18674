// Fused QK RMSNorm + 3-D RoPE kernels with e4m3fn outputs, both pairings, every row tier.
#include "dn_rope_instantiate.h"

namespace dn {
template hipError_t rope_launch<false, true>(const RopeParams&, int, int, size_t, hipStream_t,
                                           const void**);
template hipError_t rope_launch<true, true>(const RopeParams&, int, int, size_t, hipStream_t,
                                          const void**);
}  // namespace dn
