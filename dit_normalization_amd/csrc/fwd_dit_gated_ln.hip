// Forward kernels: input kind IN_GATED_BIAS, epilogue EPI_LN_BF16, every row tier.
#include "dn_fwd_instantiate.h"

namespace dn {
template hipError_t fwd_launch<IN_GATED_BIAS, EPI_LN_BF16>(
    const FwdParams&, int, int, size_t, hipStream_t, const void**);
}  // namespace dn
