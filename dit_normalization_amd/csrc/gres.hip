// Gated-residual RMSNorm kernels (with and without the next RMSNorm), every row tier.
#include "dn_launch.h"

namespace dn {

template <bool NEXT>
hipError_t gres_launch(const GresParams& p, int tier, int grid, size_t lds, hipStream_t s,
                       const void** kernel_out) {
  switch (tier) {
#define DN_X(i, tpr, v, r, nt)                                                       \
  case i:                                                                           \
    if constexpr (v <= 6) {                                                         \
      auto k = gres_kernel<tpr, v, r, nt, NEXT>;                                    \
      if (kernel_out) {                                                             \
        *kernel_out = reinterpret_cast<const void*>(k);                             \
        return hipSuccess;                                                          \
      }                                                                             \
      hipLaunchKernelGGL(k, dim3(grid), dim3(nt), lds, s, p);                       \
      return hipGetLastError();                                                     \
    } else {                                                                        \
      return hipErrorInvalidValue;                                                  \
    }
    DN_FWD_TIERS(DN_X)
#undef DN_X
    default:
      return hipErrorInvalidValue;
  }
}

template hipError_t gres_launch<false>(const GresParams&, int, int, size_t, hipStream_t,
                                       const void**);
template hipError_t gres_launch<true>(const GresParams&, int, int, size_t, hipStream_t,
                                      const void**);

}  // namespace dn
