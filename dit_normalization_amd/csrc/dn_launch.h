// Host-side launch interface between the C-ABI layer (abi.hip) and the translation units
// that instantiate the kernels (fwd_*.hip, bwd.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "dn_bwd.h"
#include "dn_fwd.h"
#include "dn_gres.h"
#include "dn_rope.h"

namespace dn {

struct TierShape {
  int tpr, vmax, r, nt;
};

// Forward tier table in host form (mirrors DN_FWD_TIERS).
inline TierShape fwd_tier_shape(int tier) {
  switch (tier) {
#define DN_X(i, tpr, v, r, nt) \
  case i: return TierShape{tpr, v, r, nt};
    DN_FWD_TIERS(DN_X)
#undef DN_X
  }
  return TierShape{0, 0, 0, 0};
}

inline TierShape bwd_tier_shape(int tier) {
  switch (tier) {
#define DN_X(i, tpr, v, r, nt) \
  case i: return TierShape{tpr, v, r, nt};
    DN_BWD_TIERS(DN_X)
#undef DN_X
  }
  return TierShape{0, 0, 0, 0};
}

// Launch one forward kernel instance (IN, EPI) of the given tier.  Returns the HIP error
// of the launch.  `kernel_out`, when non-null, receives the kernel's address instead of
// launching (used for occupancy queries).
template <int IN, int EPI>
hipError_t fwd_launch(const FwdParams& p, int tier, int grid, size_t lds, hipStream_t s,
                      const void** kernel_out);

inline TierShape rope_tier_shape(int tier) {
  switch (tier) {
#define DN_X(i, tpr, v, nt) \
  case i: return TierShape{tpr, v, 1, nt};
    DN_ROPE_TIERS(DN_X)
#undef DN_X
  }
  return TierShape{0, 0, 0, 0};
}

// Launch one fused QK RMSNorm + RoPE kernel instance (or return its address).
template <bool NEOX, bool FP8>
hipError_t rope_launch(const RopeParams& p, int tier, int grid, size_t lds, hipStream_t s,
                       const void** kernel_out);

// Launch one gated-residual RMSNorm kernel instance (forward tier table, VMAX <= 6).
template <bool NEXT>
hipError_t gres_launch(const GresParams& p, int tier, int grid, size_t lds, hipStream_t s,
                       const void** kernel_out);

hipError_t bwd_partials_launch(const BwdParams& p, int tier, size_t lds, hipStream_t s,
                               const void** kernel_out);
hipError_t bwd_reduce_launch(void* dw, int dw_bf16, const double* part, int hidden,
                             int chunks, hipStream_t s);

}  // namespace dn
