// Device helpers for the gfx950 RMSNorm kernels: BF16 / FP8 packing, 16-byte row access,
// and lane-group reductions.  Everything here is written for CDNA4 wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

// 16-byte and 8-byte register vectors (clang ext-vectors: usable in any address space).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ BF16 packing
// A 16-byte vector holds 8 BF16 values: 4 dwords, each a pair (low half = even element).

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const v4u& v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two FP32 values to a BF16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// Hides a packed vector's value from the optimiser so that a later pass unpacks it again
// (two VALU ops per pair) instead of keeping eight unpacked FP32 values live across a
// reduction: halves the row's register footprint.
__device__ __forceinline__ void keep_packed(v4u& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ v4u pack8(const float f[8]) {
  v4u v;
  v.x = pack_bf16x2(f[0], f[1]);
  v.y = pack_bf16x2(f[2], f[3]);
  v.z = pack_bf16x2(f[4], f[5]);
  v.w = pack_bf16x2(f[6], f[7]);
  return v;
}

// ------------------------------------------------------------------ FP8 e4m3fn packing
// Largest finite e4m3fn magnitude; inputs are clamped to it first so every out-of-range
// value saturates (v_med3_f32), then converted with round-to-nearest-even
// (v_cvt_pk_fp8_f32: two values into one 16-bit half of a dword, first operand in the
// lower byte).  The clamp follows IEEE minNum/maxNum and would turn a NaN into a finite
// value, so NaN bypasses it and converts to the e4m3fn NaN.
constexpr float kE4M3Max = 448.0f;

// kNanSafe = false drops the NaN bypass, for callers that have established that no
// value can be NaN (finite inputs, statistics and parameters).
template <bool kNanSafe = true>
__device__ __forceinline__ float clamp_e4m3(float v) {
  const float c = __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max);
  if constexpr (kNanSafe) return v == v ? c : v;
  return c;
}

template <bool kNanSafe = true>
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3<kNanSafe>(a), clamp_e4m3<kNanSafe>(b), 0,
                                          false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3<kNanSafe>(c), clamp_e4m3<kNanSafe>(d), r,
                                      true);
  return (uint32_t)r;
}

template <bool kNanSafe = true>
__device__ __forceinline__ v2u pack_fp8x8(const float f[8]) {
  v2u v;
  v.x = pack_fp8x4<kNanSafe>(f[0], f[1], f[2], f[3]);
  v.y = pack_fp8x4<kNanSafe>(f[4], f[5], f[6], f[7]);
  return v;
}

// The same codes for values the caller has shown to lie within [-448, 448] (NaN passes
// through as the NaN code either way): the clamp is the identity there and is left out.
__device__ __forceinline__ v2u pack_fp8x8_in_range(const float f[8]) {
  v2u v;
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  v.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], r, true);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  v.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], r, true);
  return v;
}

// pack_fp8x8<true> codes of values the caller bounds by `lim` <= 448 where it can: when
// no lane of the wave holds a magnitude above `lim` (a vote; the running maximum skips
// NaN, which converts to the NaN code either way) the clamp is left out.
__device__ __forceinline__ v2u pack_fp8x8_voted(const float f[8], float lim) {
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(f[k]));
  if (__builtin_amdgcn_ballot_w64(!(am <= lim)) == 0) return pack_fp8x8_in_range(f);
  return pack_fp8x8(f);
}

// ------------------------------------------------------------------ memory access
// Rows are read and written through raw buffer descriptors (SGPRs): the descriptor's base
// is the first row a wave touches and its record count bounds the bytes that belong to
// the rows in flight.  Each access needs one 32-bit per-lane offset; the hardware range
// check returns zeros for loads past the bound and drops stores past it, which is how
// ragged row tails and rows beyond the matrix are handled without branches.

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Descriptor word 3 for a raw (unswizzled, stride 0) buffer of 32-bit data on gfx9-family
// parts (CDNA included).
constexpr int kRawBufferWord3 = 0x00020000;

// A per-lane offset that no descriptor built here reaches (record counts stay below 2^30).
constexpr uint32_t kOutOfRange = 0x7ffffff0u;

// Cache policy of streamed rows (the buffer instructions' cache-policy operand: bit 0 sc0,
// bit 1 nt, bit 4 sc1).  Every activation byte is touched once, so rows are loaded and
// stored non-temporally: on MI355X this lifts a streaming read from ~4.6 to ~6.9 TB/s and a
// read+write copy from ~4.9 to ~5.9 TB/s (measured), where temporal hints only churn the
// caches.  Row stores also carry device scope (sc1): they leave no dirty lines in an
// XCD's L2 to be written back later (each such store covers whole 128-byte lines), which
// measured +4.7 % on the fused add [8192,4096], +3.2 % with its static FP8 output, +1.3 %
// on the training backward and on block FP8, -0.6 % on the training forward, and within
// +-1.2 % on the other families (60 and 40 interleaved launches).  Side arrays written a
// few bytes at a time (rstd, block scales) keep the default policy: their lines fill in L2
// from many stores; the backward's chunk rows take device scope alone (dn_bwd.h).
#ifndef DN_LOAD_POLICY
#define DN_LOAD_POLICY 2
#endif
#ifndef DN_STORE_POLICY
#define DN_STORE_POLICY 18
#endif
constexpr int kLoadPolicy = DN_LOAD_POLICY;
constexpr int kStorePolicy = DN_STORE_POLICY;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRawBufferWord3);
}

__device__ __forceinline__ v4u bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadPolicy));
}
// Temporal load: for data every row reads again (a broadcast style row).
__device__ __forceinline__ v4u bload16_keep(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, const v4u& v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off,
      0, kStorePolicy);
}
// Stores with an explicit cache policy (the backward's chunk rows, see dn_bwd.h).
template <int POLICY>
__device__ __forceinline__ void bstore16_p(rsrc_t r, uint32_t off, const v4u& v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off,
      0, POLICY);
}
template <int POLICY>
__device__ __forceinline__ void bstore8_p(rsrc_t r, uint32_t off, const v2u& v) {
  __builtin_amdgcn_raw_buffer_store_b64(
      __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, off,
      0, POLICY);
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, const v2u& v) {
  __builtin_amdgcn_raw_buffer_store_b64(
      __builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, off,
      0, kStorePolicy);
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Plain (flat) accesses for small side arrays (weights, per-row scalars).
__device__ __forceinline__ v4u ld16(const uint16_t* p) {
  return *reinterpret_cast<const v4u*>(p);
}

// Row-group geometry shared by the forward and backward kernels.
//   TPR threads own one row; a block of NT threads has G = NT/TPR row groups and each
//   walks R rows per step.  When TPR < 64 a wave holds RPW = 64/TPR rows side by side
//   and takes R*RPW consecutive rows per step; when TPR >= 64 a group takes R
//   consecutive rows, one per row slot.
template <int TPR, int R, int NT>
struct RowGeom {
  static constexpr int G = NT / TPR;
  static constexpr int RPW = TPR < 64 ? 64 / TPR : 1;
  static constexpr int WPR = TPR > 64 ? TPR / 64 : 1;
  static constexpr int PER_ITER = G * R;
  int lane;   // column lane inside the row group, 0..TPR-1
  int j;      // row slot inside the wave (TPR < 64), else 0
  int grp;    // row group (wave-uniform when TPR >= 64)
  int wave;   // wave inside the block (uniform)
  __device__ __forceinline__ RowGeom() {
    const int tid = threadIdx.x;
    lane = tid % TPR;
    j = TPR < 64 ? (tid & 63) / TPR : 0;
    wave = wave_uniform(tid >> 6);
    grp = TPR >= 64 ? wave_uniform(tid / TPR) : tid / TPR;
  }
  // First row of the span this wave (TPR < 64) or row group (TPR >= 64) owns in a step.
  __device__ __forceinline__ int64_t first(int64_t base) const {
    return TPR < 64 ? base + (int64_t)wave * R * RPW : base + (int64_t)grp * R;
  }
  // Row slot rr of this lane.
  __device__ __forceinline__ int64_t row(int64_t first_row, int rr) const {
    return TPR < 64 ? first_row + rr * RPW + j : first_row + rr;
  }
};

// Buffer descriptors and lane offsets of one row-major tensor for the R row slots of a
// step.  `elem` is the element size, `vec` the bytes one lane moves per access (16 for
// BF16 vectors, 8 for FP8), `span` the bytes of a row that belong to it, `end` the first
// row that must not be touched, and `lane_ok` false for lanes past the row's last vector.
template <int TPR, int R, int RPW>
__device__ __forceinline__ void tensor_span(const void* t, int64_t stride, int elem, int vec,
                                            uint32_t span, int64_t first, int64_t end,
                                            int lane, int j, bool lane_ok, rsrc_t (&rs)[R],
                                            uint32_t (&off)[R]) {
  const char* base = static_cast<const char*>(t);
  if constexpr (TPR < 64) {
    int64_t nvalid = end - first;
    nvalid = nvalid < 0 ? 0 : (nvalid > R * RPW ? R * RPW : nvalid);
    const rsrc_t r = make_rsrc(base + first * stride * elem, (uint32_t)(nvalid * stride * elem));
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      rs[rr] = r;
      off[rr] = lane_ok ? (uint32_t)((rr * RPW + j) * stride * elem) + (uint32_t)(lane * vec)
                        : kOutOfRange;
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int64_t row = first + rr;
      rs[rr] = make_rsrc(base + row * stride * elem, row < end ? span : 0u);
      off[rr] = (uint32_t)(lane * vec);
    }
  }
}

// ------------------------------------------------------------------ sums of squares
// Squares of BF16 values are exact in FP32.  Eight of them are added as a 3-level tree
// (every product passes through at most three FP32 roundings, relative error <= 3*2^-24),
// and the per-vector sums are carried in FP64 from there on.
__device__ __forceinline__ float sumsq8(const float f[8]) {
  float s01 = fmaf(f[1], f[1], f[0] * f[0]);
  float s23 = fmaf(f[3], f[3], f[2] * f[2]);
  float s45 = fmaf(f[5], f[5], f[4] * f[4]);
  float s67 = fmaf(f[7], f[7], f[6] * f[6]);
  return (s01 + s23) + (s45 + s67);
}

// The same sum carried to FP64, safe for any BF16 input.  Two cases make the FP32 tree
// not good enough: an FP32 square or the tree overflows (|value| above ~6.5e18; no
// realistic activation), or `exact` is set by the caller because eps is so small (below
// 2^-80) that squares lost to FP32 underflow could matter next to it.  Then the eight
// squares are summed in FP64 (exact products).  The test is a wave vote, so the FP64 sum
// is a branch the wave skips unless one of its lanes needs it; a per-lane select would
// make every lane pay for both sums (measured: -10 % on the VALU-heavy SiLU rows).
//
// kJointVote votes on `exact || overflow` instead, which makes the compiler carry the mask
// through a VGPR (two more VALU instructions per call) and schedules the surrounding code
// differently: measured 2-3 % faster in the NeoX QK RoPE kernel with BF16 outputs (two
// waves per SIMD), 2 % slower with FP8 outputs and no different elsewhere, so only that
// instance asks for it.  Both forms give the same sums.
template <bool kJointVote = false>
__device__ __forceinline__ double sumsq8_d(const float f[8], bool exact) {
  const float t = sumsq8(f);
  if constexpr (kJointVote) {
    const bool redo = exact || !(t <= 3.0e38f);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(redo) == 0, 1)) return (double)t;
    asm volatile("");   // keeps the FP64 sum behind the branch
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = fma((double)f[k], (double)f[k], s);
    return redo ? s : (double)t;
  }
  // `exact` lowers the limit below every sum (then every lane takes the FP64 sum), so the
  // comparison feeds the vote alone and the vote is its lane mask as it stands.  (Voting
  // on `exact || big`, or using the comparison past the branch, makes the compiler carry
  // the mask through a VGPR: two more VALU instructions per call.)
  const float limit = exact ? -1.0f : 3.0e38f;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(t <= limit)) == 0, 1)) return (double)t;
  // The empty volatile statement keeps the compiler from hoisting this block above the
  // branch (it would otherwise evaluate both sums and select), and hides `t` from it, so
  // the lane's comparison below is made afresh instead of carried past the branch.
  float tt = t;
  asm volatile("" : "+v"(tt));
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) s = fma((double)f[k], (double)f[k], s);
  return !(tt <= limit) ? s : (double)tt;
}

// FP32(a / 448) for a >= 0 the value of a BF16 number (a block's largest |n|), correctly
// rounded, in one multiply and two FMAs: q0 = a * RN(1/448), r = a - 448 q0 (exact in one
// FMA), q = q0 + r * RN(1/448).  One correction step of this kind is not correctly rounded
// for every FP32 input, but it is for every BF16 input: checked exhaustively with exact
// rational arithmetic over all 32,639 positive finite BF16 values, subnormals included
// (the unit test of this identity sits with the host tests).
__device__ __forceinline__ float div_by_448(float a) {
  constexpr float kInv448 = 1.0f / 448.0f;
  const float q0 = a * kInv448;
  const float r = fmaf(-q0, 448.0f, a);
  return fmaf(r, kInv448, q0);
}

// ------------------------------------------------------------------ cross-lane sums
// Partner exchanges on the VALU only, no LDS round trip: DPP quad permutations and row
// mirrors inside a 16-lane row, and gfx950's permute-swap instructions between rows (they
// hand both lanes of a lane ^ 16 or lane ^ 32 pair the pair's two values, lower lane first).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ double make_f64(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Step M (1, 2, 4, 8, 16, 32) of a group sum: v plus the value of the partner lane, where
// after steps 1 .. M/2 every lane holds the sum of its aligned group of M lanes and the
// partner holds the sum of the neighbouring group: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror, then the row swaps.  Both lanes of a pair add the
// same two operands (addition commutes), so the whole group ends with the same bits.
template <int M>
__device__ __forceinline__ double add_partner(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  if constexpr (M <= 8) {
    constexpr int C = M == 1 ? 0xB1 : (M == 2 ? 0x4E : (M == 4 ? 0x141 : 0x140));
    return v + make_f64(dpp_u32<C>(lo), dpp_u32<C>(hi));
  } else if constexpr (M == 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    return make_f64(a[0], b[0]) + make_f64(a[1], b[1]);
  } else {
    static_assert(M == 32, "group steps go up to 32");
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    return make_f64(a[0], b[0]) + make_f64(a[1], b[1]);
  }
}

// Sum over aligned groups of WIDTH lanes (WIDTH a power of two <= 64); every lane of a
// group ends with the same bits.
template <int WIDTH>
__device__ __forceinline__ double group_sum(double v) {
  static_assert(WIDTH >= 1 && WIDTH <= 64 && (WIDTH & (WIDTH - 1)) == 0, "power of two");
  if constexpr (WIDTH >= 2) v = add_partner<1>(v);
  if constexpr (WIDTH >= 4) v = add_partner<2>(v);
  if constexpr (WIDTH >= 8) v = add_partner<4>(v);
  if constexpr (WIDTH >= 16) v = add_partner<8>(v);
  if constexpr (WIDTH >= 32) v = add_partner<16>(v);
  if constexpr (WIDTH >= 64) v = add_partner<32>(v);
  return v;
}

// FP32(1 / sqrt(x)) for the statistics: the hardware FP64 reciprocal square root (relative
// error below 2^-24, measured) refined by two Newton steps (below 2^-52, measured over 4M
// inputs spanning 1e-300 .. 1e301), as close as an IEEE square root followed by an IEEE
// divide, for a fraction of their instructions.  Inputs outside [2^-1000, 2^1000], zero,
// infinity and NaN included, take the IEEE path; the test is a wave vote, so the wave
// branches round it unless one of its lanes needs it.
__device__ __forceinline__ double rsqrt_f64(double x) {
  const bool plain = x >= 0x1p-1000 && x <= 0x1p1000;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(!plain) == 0, 1)) {
    double y = __builtin_amdgcn_rsq(x);
    y = fma(0.5 * y, fma(-x * y, y, 1.0), y);
    y = fma(0.5 * y, fma(-x * y, y, 1.0), y);
    return y;
  }
  asm volatile("");   // keeps the IEEE path behind the branch, not evaluated and selected
  return 1.0 / sqrt(x);
}

// Maximum over each aligned group of 16 lanes (one DPP row) of values that are >= +0 and
// not NaN, with four DPP steps and no LDS traffic: swap neighbours, swap pairs (quad
// permutations), then mirror each half row and the whole row; after each step every lane
// holds the maximum of twice as many lanes.  For such values IEEE order is the order of
// their bit patterns as unsigned integers, so each step is a DPP move and an integer
// maximum (a float maximum would first quiet the moved operand: one more instruction per
// step).
__device__ __forceinline__ float row16_max(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t t = dpp_u32<0xB1>(u);    // quad_perm [1, 0, 3, 2]
  u = u > t ? u : t;
  t = dpp_u32<0x4E>(u);             // quad_perm [2, 3, 0, 1]
  u = u > t ? u : t;
  t = dpp_u32<0x141>(u);            // row_half_mirror
  u = u > t ? u : t;
  t = dpp_u32<0x140>(u);            // row_mirror
  u = u > t ? u : t;
  return __uint_as_float(u);
}

// Maximum of two results of arithmetic (never signalling NaNs) as one v_max_f32: IEEE
// maxNum, so a NaN operand yields the other one, the same as fmaxf, without the quieting
// pass the compiler puts in front of fmaxf operands it cannot prove canonical (one extra
// instruction per value).  The compiler's hazard checks cannot be relied on to see a
// register written by inline assembly, so the result is never fed to a DPP move.
__device__ __forceinline__ float max_of_results(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

}  // namespace dn
