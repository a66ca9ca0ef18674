// Training-backward kernels: the producers (dx and per-chunk FP64 column sums) over every
// row tier, and the fixed-order dw reduction.
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

hipError_t bwd_reduce_launch(void* dw, int dw_bf16, const double* part, int hidden,
                             int chunks, hipStream_t s) {
  const int grid = (hidden + kReduceCols - 1) / kReduceCols;
  hipLaunchKernelGGL(bwd_reduce_kernel<kReduceThreads>, dim3(grid), dim3(kReduceThreads), 0, s, dw, dw_bf16,
                     part, hidden, chunks);
  return hipGetLastError();
}

}  // namespace dn
