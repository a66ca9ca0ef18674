// Forward kernels: input kind IN_PLAIN, epilogue EPI_SILU_FP8, every row tier.
#include "dn_fwd_instantiate.h"

namespace dn {
template hipError_t fwd_launch<IN_PLAIN, EPI_SILU_FP8>(
    const FwdParams&, int, int, size_t, hipStream_t, const void**);
}  // namespace dn
