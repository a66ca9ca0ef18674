// Training-backward kernels: stage 1 over every row tier, and the fixed-order dw reduction.
#include "dn_launch.h"

namespace dn {

hipError_t bwd_partials_launch(const BwdParams& p, int tier, size_t lds, hipStream_t s,
                               const void** kernel_out) {
  switch (tier) {
#define DN_X(i, tpr, v, r, nt)                                                       \
  case i: {                                                                         \
    auto k = p.gres ? bwd_partials_kernel<tpr, v, r, nt, true>                      \
                    : bwd_partials_kernel<tpr, v, r, nt, false>;                    \
    if (kernel_out) {                                                               \
      *kernel_out = reinterpret_cast<const void*>(k);                               \
      return hipSuccess;                                                            \
    }                                                                               \
    hipLaunchKernelGGL(k, dim3(p.chunks), dim3(nt), lds, s, p);                     \
    return hipGetLastError();                                                       \
  }
    DN_BWD_TIERS(DN_X)
#undef DN_X
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t bwd_reduce_launch(float* dw, const double* part, int hidden, int chunks,
                             hipStream_t s) {
  constexpr int NT = 512;
  const int grid = (hidden + 63) / 64;
  hipLaunchKernelGGL(bwd_reduce_kernel<NT>, dim3(grid), dim3(NT), 0, s, dw, part, hidden,
                     chunks);
  return hipGetLastError();
}

}  // namespace dn
