// HBM stream ceilings of MI355X for the read:write mixes of the norm kernels.
//
// A measurement aid, not part of the norm library: bench.py loads it (libdnprobe.so) to
// report what a plain streaming kernel reaches with the same memory instructions (16-byte
// non-temporal buffer loads and stores) and the same read:write mixes as the norm kernels
// (1 read : 1 write, 2 : 2, 2 : 1, 3 : 1).  Each lane streams 16-byte vectors; the value
// written is a function of the values read, so no load can be dropped.
//
// Access strategies (`mode`):
//   0  grid-stride: each lane takes 4 vectors per round, rounds dealt over the whole grid
//      (the norm kernels' pattern);
//   1  contiguous chunks: block b streams its own contiguous 1/grid of every buffer;
//   2  XCD partition: the blocks of each of the 8 XCDs (dealt round-robin) stream one
//      contiguous eighth of every buffer, grid-stride inside it;
//   3  LDS pipeline: 16-byte loads go straight into LDS (no VGPRs held), kPipe rounds of
//      every source in flight per wave; a round's values are read back and stored;
//   4  block phases: each block reads kPhase rounds of every source (through registers
//      into LDS), then writes them all: long read phases and long write phases per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dn_device.h"

using namespace dn;

namespace {

constexpr int kPipe = 6;    // mode 3: rounds in flight per wave (the first-pass waits below
                            // are written out for 6)
constexpr int kPhase = 4;   // mode 4: rounds per phase (4 vectors per lane per round); 2
                            // with three sources (LDS holds at most 160 KiB)

template <int NR, int NW>
__device__ __forceinline__ void store_round(const rsrc_t& w0, const rsrc_t& w1, uint32_t off,
                                            const v4u& a, const v4u& b, const v4u& c) {
  v4u o = a;
  if constexpr (NR > 1) o ^= b;
  if constexpr (NR > 2) o ^= c;
  bstore16(w0, off, o);
  if constexpr (NW > 1) bstore16(w1, off, o + a);
}

// Modes 0-2: registers only, 4 vectors per lane per round.
template <int NR, int NW>
__global__ void __launch_bounds__(256) stream_kernel(const uint8_t* s0, const uint8_t* s1,
                                                     const uint8_t* s2, uint8_t* d0,
                                                     uint8_t* d1, uint32_t bytes, int mode) {
  const rsrc_t r0 = make_rsrc(s0, bytes), r1 = make_rsrc(s1, NR > 1 ? bytes : 0u),
               r2 = make_rsrc(s2, NR > 2 ? bytes : 0u);
  const rsrc_t w0 = make_rsrc(d0, bytes), w1 = make_rsrc(d1, NW > 1 ? bytes : 0u);
  const uint32_t nvec = bytes / 16u;
  uint32_t start, end, stride;
  if (mode == 1) {
    const uint32_t per_block = (nvec + gridDim.x - 1) / gridDim.x;
    start = blockIdx.x * per_block;
    end = min(start + per_block, nvec);
    stride = 256u;
  } else if (mode == 2) {
    const uint32_t xcd = blockIdx.x & 7u, nb = gridDim.x >> 3;   // grid % 8 == 0
    const uint32_t per_xcd = (nvec + 7u) / 8u;
    start = xcd * per_xcd + (blockIdx.x >> 3) * 256u;
    end = min((xcd + 1u) * per_xcd, nvec);
    stride = nb * 256u;
  } else {
    start = blockIdx.x * 256u;
    end = nvec;
    stride = gridDim.x * 256u;
  }
  const uint32_t step = mode == 1 ? 256u * 4u : stride * 4u;
  for (uint32_t base = start + threadIdx.x; base < end; base += step) {
    v4u a[4], b[4], c[4];
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
      store_round<NR, NW>(w0, w1, i < end ? i * 16u : kOutOfRange, a[k], b[k], c[k]);
    }
  }
}

// Mode 3: a wave's round is 64 consecutive vectors (1 KiB) of every source; rounds are
// dealt over all waves of the grid.  Round j of a wave lands in LDS slot j % kPipe.  The
// loop is unrolled by kPipe so every slot is a fixed LDS address.
template <int NR, int NW>
__global__ void __launch_bounds__(256) lds_pipe_kernel(const uint8_t* s0, const uint8_t* s1,
                                                       const uint8_t* s2, uint8_t* d0,
                                                       uint8_t* d1, uint32_t bytes) {
  __shared__ __align__(16) unsigned char lds[4][kPipe][NR][1024];
  const rsrc_t r0 = make_rsrc(s0, bytes), r1 = make_rsrc(s1, NR > 1 ? bytes : 0u),
               r2 = make_rsrc(s2, NR > 2 ? bytes : 0u);
  const rsrc_t w0 = make_rsrc(d0, bytes), w1 = make_rsrc(d1, NW > 1 ? bytes : 0u);
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  const uint32_t nvec = bytes / 16u;
  const uint32_t gw = blockIdx.x * 4u + wave, tw = gridDim.x * 4u;
  const uint32_t rounds = (nvec + 63u) / 64u;
  auto off_of = [&](uint32_t j) -> uint32_t {   // byte offset of this lane in round j
    const uint32_t u = gw + j * tw;
    const uint32_t v = u * 64u + lane;
    return u < rounds && v < nvec ? v * 16u : kOutOfRange;
  };
  auto issue = [&](uint32_t j, int slot) {
    const uint32_t off = off_of(j);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r0, (__attribute__((address_space(3))) void*)&lds[wave][slot][0][0], 16, off, 0, 0, 2);
    if constexpr (NR > 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r1, (__attribute__((address_space(3))) void*)&lds[wave][slot][1][0], 16, off, 0, 0,
          2);
    if constexpr (NR > 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r2, (__attribute__((address_space(3))) void*)&lds[wave][slot][2][0], 16, off, 0, 0,
          2);
  };
  const uint32_t my_rounds = gw < rounds ? (rounds - gw + tw - 1) / tw : 0u;
#pragma unroll
  for (int s = 0; s < kPipe; ++s) issue(s, s);
  // Iteration j: wait for round j, read it from its slot, refill the slot with round
  // j + kPipe, store round j (stores past the data are issued too, dropped by the range
  // check, so every iteration issues the same operations).  Vector memory operations
  // complete in issue order for the counter, so round j has landed once no more than the
  // operations issued after it are outstanding: (kPipe-1-j)*NR + j*(NR+NW) in the first
  // kPipe iterations, NW + (kPipe-1)*(NR+NW) after.
  auto body = [&](uint32_t j, int s, auto n_after) {
    constexpr int N = decltype(n_after)::value;
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    const v4u a = *reinterpret_cast<const v4u*>(&lds[wave][s][0][lane * 16]);
    v4u b = a, c = a;
    if constexpr (NR > 1) b = *reinterpret_cast<const v4u*>(&lds[wave][s][1][lane * 16]);
    if constexpr (NR > 2) c = *reinterpret_cast<const v4u*>(&lds[wave][s][2][lane * 16]);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the slot's values are in VGPRs
    issue(j + kPipe, s);
    store_round<NR, NW>(w0, w1, off_of(j), a, b, c);
  };
  constexpr int kSteady = NW + (kPipe - 1) * (NR + NW);
  static_assert(kSteady < 64, "vmcnt holds 6 bits");
  if (my_rounds > 0) {
    body(0, 0, std::integral_constant<int, (kPipe - 1) * NR>{});
    body(1, 1, std::integral_constant<int, (kPipe - 2) * NR + 1 * (NR + NW)>{});
    body(2, 2, std::integral_constant<int, (kPipe - 3) * NR + 2 * (NR + NW)>{});
    body(3, 3, std::integral_constant<int, (kPipe - 4) * NR + 3 * (NR + NW)>{});
    body(4, 4, std::integral_constant<int, (kPipe - 5) * NR + 4 * (NR + NW)>{});
    body(5, 5, std::integral_constant<int, (kPipe - 6) * NR + 5 * (NR + NW)>{});
  }
  for (uint32_t j0 = kPipe; j0 < my_rounds; j0 += kPipe) {
#pragma unroll
    for (int s = 0; s < kPipe; ++s) body(j0 + s, s, std::integral_constant<int, kSteady>{});
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Mode 4: a block takes kPhase rounds of 4 vectors per lane (1024 consecutive vectors of
// every source per round), reads them all into LDS, then writes them all.
template <int NR, int NW>
__global__ void __launch_bounds__(256) phase_kernel(const uint8_t* s0, const uint8_t* s1,
                                                    const uint8_t* s2, uint8_t* d0,
                                                    uint8_t* d1, uint32_t bytes) {
  constexpr int P = NR > 2 ? 2 : kPhase;
  __shared__ __align__(16) v4u lds[P][NR][1024];
  const rsrc_t r0 = make_rsrc(s0, bytes), r1 = make_rsrc(s1, NR > 1 ? bytes : 0u),
               r2 = make_rsrc(s2, NR > 2 ? bytes : 0u);
  const rsrc_t w0 = make_rsrc(d0, bytes), w1 = make_rsrc(d1, NW > 1 ? bytes : 0u);
  const uint32_t nvec = bytes / 16u;
  const uint32_t per_phase = P * 1024u;
  for (uint32_t base = blockIdx.x * per_phase; base < nvec; base += gridDim.x * per_phase) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t e = p * 1024u + k * 256u + threadIdx.x;
        const uint32_t i = base + e;
        const uint32_t off = i < nvec ? i * 16u : kOutOfRange;
        lds[p][0][k * 256u + threadIdx.x] = bload16(r0, off);
        if constexpr (NR > 1) lds[p][1][k * 256u + threadIdx.x] = bload16(r1, off);
        if constexpr (NR > 2) lds[p][2][k * 256u + threadIdx.x] = bload16(r2, off);
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t e = k * 256u + threadIdx.x;
        const uint32_t i = base + p * 1024u + e;
        const v4u a = lds[p][0][e];
        const v4u b = NR > 1 ? lds[p][NR > 1 ? 1 : 0][e] : a;
        const v4u c = NR > 2 ? lds[p][NR > 2 ? 2 : 0][e] : a;
        store_round<NR, NW>(w0, w1, i < nvec ? i * 16u : kOutOfRange, a, b, c);
      }
    }
    __syncthreads();
  }
}

template <int NR, int NW>
int launch(const uint8_t* a, const uint8_t* b, const uint8_t* c, uint8_t* x, uint8_t* y,
           uint32_t n, int blocks, int mode, hipStream_t st) {
  const dim3 g(blocks), t(256);
  if (mode <= 2)
    hipLaunchKernelGGL((stream_kernel<NR, NW>), g, t, 0, st, a, b, c, x, y, n, mode);
  else if (mode == 3)
    hipLaunchKernelGGL((lds_pipe_kernel<NR, NW>), g, t, 0, st, a, b, c, x, y, n);
  else
    hipLaunchKernelGGL((phase_kernel<NR, NW>), g, t, 0, st, a, b, c, x, y, n);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // namespace

extern "C" {

// reads: 1, 2 or 3 source buffers; writes: 1 or 2 destinations; all `bytes` long (a
// multiple of 16, below 2^31).  blocks: grid size (a multiple of 8 for mode 2); mode: the
// access strategy above.  Returns 0, or -1 for an unsupported argument, -2 for a failed
// launch.
int dn_probe_stream(const void* s0, const void* s1, const void* s2, void* d0, void* d1,
                    int64_t bytes, int reads, int writes, int blocks, int mode,
                    void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || bytes >= ((int64_t)1 << 31) || blocks <= 0) return -1;
  if (mode < 0 || mode > 4 || (mode == 2 && blocks % 8 != 0)) return -1;
  const auto* a = static_cast<const uint8_t*>(s0);
  const auto* b = static_cast<const uint8_t*>(s1);
  const auto* c = static_cast<const uint8_t*>(s2);
  auto* x = static_cast<uint8_t*>(d0);
  auto* y = static_cast<uint8_t*>(d1);
  const uint32_t n = (uint32_t)bytes;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (reads == 1 && writes == 1) return launch<1, 1>(a, b, c, x, y, n, blocks, mode, st);
  if (reads == 2 && writes == 2) return launch<2, 2>(a, b, c, x, y, n, blocks, mode, st);
  if (reads == 2 && writes == 1) return launch<2, 1>(a, b, c, x, y, n, blocks, mode, st);
  if (reads == 3 && writes == 1) return launch<3, 1>(a, b, c, x, y, n, blocks, mode, st);
  return -1;
}

}  // extern "C"
