// Forward kernels: input kind IN_ADD, epilogue EPI_FP8_BLOCK, every row tier.
#include "dn_fwd_instantiate.h"

namespace dn {
template hipError_t fwd_launch<IN_ADD, EPI_FP8_BLOCK>(const FwdParams&, int, int, size_t, hipStream_t,
                                       const void**);
}  // namespace dn
