// Definition of fwd_launch<IN, EPI>, included by the fwd_*.hip units only: each unit
// instantiates one (input, epilogue) combination over every row tier it is built with.
#pragma once

#include "dn_launch.h"

namespace dn {

template <int IN, int EPI>
hipError_t fwd_launch(const FwdParams& p, int tier, int grid, size_t lds, hipStream_t s,
                      const void** kernel_out) {
  switch (tier) {
#define DN_X(i, tpr, v, r, nt)                                                       \
  case i:                                                                           \
    if constexpr (v <= fwd_vmax_limit(IN, EPI)) {                                   \
      auto k = fwd_kernel<IN, EPI, tpr, v, r, nt>;                                  \
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

}  // namespace dn
