// Forward kernels: input kind IN_PLAIN, epilogue EPI_SIGMOID_GATE, every row tier.
#include "dn_fwd_instantiate.h"

namespace dn {
template hipError_t fwd_launch<IN_PLAIN, EPI_SIGMOID_GATE>(
    const FwdParams&, int, int, size_t, hipStream_t, const void**);
}  // namespace dn
