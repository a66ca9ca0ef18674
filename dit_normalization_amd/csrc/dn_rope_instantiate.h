// Definition of rope_launch<NEOX, FP8>, included by the rope_*.hip units only.
#pragma once

#include "dn_launch.h"

namespace dn {

template <bool NEOX, bool FP8>
hipError_t rope_launch(const RopeParams& p, int tier, int grid, size_t lds, hipStream_t s,
                       const void** kernel_out) {
  switch (tier) {
#define DN_X(i, tpr, v, nt)                                                          \
  case i: {                                                                         \
    auto k = qkrope_kernel<tpr, v, nt, NEOX, FP8>;                                  \
    if (kernel_out) {                                                               \
      *kernel_out = reinterpret_cast<const void*>(k);                               \
      return hipSuccess;                                                            \
    }                                                                               \
    hipLaunchKernelGGL(k, dim3(grid), dim3(nt), lds, s, p);                         \
    return hipGetLastError();                                                       \
  }
    DN_ROPE_TIERS(DN_X)
#undef DN_X
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dn
