// HBM stream ceilings of MI355X for the read:write mixes of the norm kernels.
//
// A measurement aid, not part of the norm library: bench.py loads it (libdnprobe.so) to
// report what a plain streaming kernel reaches with the same memory instructions (16-byte
// non-temporal buffer loads and stores) and the same read:write mixes as the norm kernels
// (1 read : 1 write, 2 : 2, 2 : 1, 3 : 1).  Each lane streams 16-byte vectors; the value
// written is a function of the values read, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dn_device.h"

using namespace dn;

namespace {

// Vectors are dealt to blocks in contiguous chunks (`blocked`: block b owns a contiguous
// range of chunk vectors per round) or round-robin per vector (grid-stride).
template <int NR, int NW>
__global__ void __launch_bounds__(256) stream_kernel(const uint8_t* s0, const uint8_t* s1,
                                                     const uint8_t* s2, uint8_t* d0,
                                                     uint8_t* d1, uint32_t bytes,
                                                     int blocked) {
  const rsrc_t r0 = make_rsrc(s0, bytes), r1 = make_rsrc(s1, NR > 1 ? bytes : 0u),
               r2 = make_rsrc(s2, NR > 2 ? bytes : 0u);
  const rsrc_t w0 = make_rsrc(d0, bytes), w1 = make_rsrc(d1, NW > 1 ? bytes : 0u);
  const uint32_t nvec = bytes / 16u;
  const uint32_t nthreads = gridDim.x * 256u;
  const uint32_t per_block = (nvec + gridDim.x - 1) / gridDim.x;
  const uint32_t start = blocked ? blockIdx.x * per_block : blockIdx.x * 256u;
  const uint32_t end = blocked ? min(start + per_block, nvec) : nvec;
  const uint32_t step = blocked ? 256u * 4u : nthreads * 4u;
  // Four vectors in flight per lane per iteration, like the norm kernels' 4 vectors per lane.
  for (uint32_t base = start + threadIdx.x; base < end; base += step) {
    v4u a[4], b[4], c[4];
    const uint32_t stride = blocked ? 256u : nthreads;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = base + k * stride;
      const uint32_t off = i < end ? i * 16u : kOutOfRange;
      a[k] = bload16(r0, off);
      if constexpr (NR > 1) b[k] = bload16(r1, off);
      if constexpr (NR > 2) c[k] = bload16(r2, off);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = base + k * stride;
      const uint32_t off = i < end ? i * 16u : kOutOfRange;
      v4u o = a[k];
      if constexpr (NR > 1) o ^= b[k];
      if constexpr (NR > 2) o ^= c[k];
      bstore16(w0, off, o);
      if constexpr (NW > 1) bstore16(w1, off, o + a[k]);
    }
  }
}

}  // namespace

extern "C" {

// reads: 1, 2 or 3 source buffers; writes: 1 or 2 destinations; all `bytes` long (a
// multiple of 16, below 2^31).  blocks: grid size; blocked: chunked (1) or grid-stride (0).
// Returns 0, or -1 for an unsupported mix, -2 for a failed launch.
int dn_probe_stream(const void* s0, const void* s1, const void* s2, void* d0, void* d1,
                    int64_t bytes, int reads, int writes, int blocks, int blocked,
                    void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || bytes >= ((int64_t)1 << 31) || blocks <= 0) return -1;
  const auto* a = static_cast<const uint8_t*>(s0);
  const auto* b = static_cast<const uint8_t*>(s1);
  const auto* c = static_cast<const uint8_t*>(s2);
  auto* x = static_cast<uint8_t*>(d0);
  auto* y = static_cast<uint8_t*>(d1);
  const uint32_t n = (uint32_t)bytes;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g(blocks), t(256);
  if (reads == 1 && writes == 1)
    hipLaunchKernelGGL((stream_kernel<1, 1>), g, t, 0, st, a, b, c, x, y, n, blocked);
  else if (reads == 2 && writes == 2)
    hipLaunchKernelGGL((stream_kernel<2, 2>), g, t, 0, st, a, b, c, x, y, n, blocked);
  else if (reads == 2 && writes == 1)
    hipLaunchKernelGGL((stream_kernel<2, 1>), g, t, 0, st, a, b, c, x, y, n, blocked);
  else if (reads == 3 && writes == 1)
    hipLaunchKernelGGL((stream_kernel<3, 1>), g, t, 0, st, a, b, c, x, y, n, blocked);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
