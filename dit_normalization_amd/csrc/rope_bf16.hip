// Fused QK RMSNorm + 3-D RoPE kernels with BF16 outputs, both pairings, every row tier.
#include "dn_rope_instantiate.h"

namespace dn {
template hipError_t rope_launch<false, false>(const RopeParams&, int, int, size_t, hipStream_t,
                                           const void**);
template hipError_t rope_launch<true, false>(const RopeParams&, int, int, size_t, hipStream_t,
                                          const void**);
}  // namespace dn
