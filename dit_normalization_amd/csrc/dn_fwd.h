// Forward row engine of the RMSNorm and LayerNorm families for gfx950.
//
// One template covers every forward variant; two compile-time kinds select what a row
// reads and what its epilogue writes:
//   input  : x | x + residual (fused add) | FMA(x, gate, residual) (gated residual) |
//            FMA(x, gate + gate_bias, residual) (DiT gated residual)
//   output : RMSNorm: BF16 y | FP8 at a static scale | FP8 with 1x128 block scales |
//            AdaRMSNorm (style scale/shift, gate copy) in BF16 or FP8
//            LayerNorm: BF16 or static FP8 of n*gamma + beta | BF16 of the DiT modulation
//            n*(1 + scale + scale_bias) + (shift + shift_bias)
//            RMSNorm + SiLU: BF16 or static FP8 of y / (1 + exp(-y))
//            RMSNorm * sigmoid(gate): BF16 of y / (1 + exp(-gate)), gate an extra row tensor
// The LayerNorm epilogues also switch the row statistics from the sum of squares to the
// FP64 pair (sum, sum of squares), from which mean and variance follow in one pass.
//
// Row mapping (chosen on the host by hidden size): a row is owned by a group of TPR
// threads.  Thread `lane` of the group owns the 16-byte column vectors lane, lane+TPR,
// lane+2*TPR, ... (VMAX of them at most), so every load instruction of a wave reads TPR
// consecutive 16-byte vectors of a row: fully coalesced.  TPR < 64 packs 64/TPR rows into
// a wave; TPR = 64 gives a wave one row; TPR > 64 spreads a row over TPR/64 waves whose
// partial sums meet in LDS.  The whole row stays in VGPRs across the reduction, so every
// input byte is read from HBM exactly once.
//
// Memory traffic goes through raw buffer descriptors (see dn_device.h): one descriptor per
// row (or per wave span of small rows) and one offset VGPR per lane; the descriptor's
// range check zero-fills ragged tails and drops their stores.
//
// Blocks are persistent: the grid is sized to the resident capacity of the chip and each
// block walks row groups with a grid stride.  Per-column parameters (the effective RMSNorm
// weight FP32(w + bias), or LayerNorm's gamma and beta) are staged once per block into
// LDS as planes of float4, so lanes read consecutive 16-byte words (conflict-free
// ds_read_b128), and read from there for every row.
#pragma once

#include "dn_device.h"

namespace dn {

enum InKind { IN_PLAIN = 0, IN_ADD = 1, IN_GATED = 2, IN_GATED_BIAS = 3 };
enum EpiKind {
  EPI_BF16 = 0, EPI_FP8 = 1, EPI_FP8_BLOCK = 2, EPI_ADA_BF16 = 3, EPI_ADA_FP8 = 4,
  EPI_LN_BF16 = 5, EPI_LN_FP8 = 6, EPI_LN_MOD_BF16 = 7, EPI_SILU_BF16 = 8, EPI_SILU_FP8 = 9,
  EPI_SIGMOID_GATE = 10
};

constexpr bool epi_is_ln(int epi) {
  return epi == EPI_LN_BF16 || epi == EPI_LN_FP8 || epi == EPI_LN_MOD_BF16;
}
constexpr bool epi_is_silu(int epi) { return epi == EPI_SILU_BF16 || epi == EPI_SILU_FP8; }
constexpr bool in_is_gated(int in) { return in == IN_GATED || in == IN_GATED_BIAS; }
// FP32 planes (16 bytes per column vector each) of per-column parameters staged in LDS:
// the RMSNorm effective weight (2), LayerNorm gamma and beta (4), none for the modulation.
constexpr int fwd_weight_planes(int epi) {
  return epi == EPI_LN_MOD_BF16 ? 0 : (epi_is_ln(epi) ? 4 : 2);
}
// FP64 statistics a row reduces: sum of squares, plus the sum for LayerNorm.
constexpr int fwd_stats(int epi) { return epi_is_ln(epi) ? 2 : 1; }

constexpr float kLog2E = 1.44269504088896341f;   // log2(e), rounded to FP32
constexpr float kLn2 = 0.693147180559945309f;    // ln(2) = 1/log2(e), rounded to FP32

struct FwdParams {
  const uint16_t* x;     int64_t sx;
  const uint16_t* r;     int64_t sr;     // residual (IN_ADD, gated inputs)
  const uint16_t* gate;  int64_t sg;     // gated inputs
  const uint16_t* style; int64_t sst;    // Ada: [style_rows, 3*hidden]
  int style_bcast;                       // Ada: one style row for every token
  const void* w;         int w_f32;      float w_bias;   // LayerNorm: w = gamma (FP32)
  const float* beta;                     // LayerNorm beta (FP32 [hidden])
  const uint16_t* msc;   int64_t smsc;   // DiT modulation scale rows (BF16)
  const uint16_t* msh;   int64_t smsh;   // DiT modulation shift rows (BF16)
  float gate_bias, scale_bias, shift_bias;
  const float* scale;                    // FP8 static: device FP32 [1]
  uint16_t* y;           int64_t sy;     // BF16 output (y, normed_out, Ada out); nullable
  uint16_t* h;           int64_t sh;     // h_new output; nullable
  uint8_t* q;            int64_t sq;     // FP8 output
  float* bscale;         int64_t bld;    // 1x128 block scales [hidden/128][bld]
  uint16_t* gate_out;    int64_t sgo;    // Ada gate copy; nullable
  float* rstd;                           // nullable
  int64_t rows;
  int hidden;
  int nvec;                              // hidden / 8
  float eps;
  int w_in_lds;                          // per-column parameters staged in LDS
};

// Effective weight FP32(w + bias) of one 16-byte column vector, read from global memory.
__device__ __forceinline__ void load_weff8(const FwdParams& p, int vec, float e[8]) {
  if (!p.w) {   // no weight: ones
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = 1.0f + p.w_bias;
    return;
  }
  if (p.w_f32) {
    const float4* w = reinterpret_cast<const float4*>(p.w) + 2 * vec;
    const float4 a = w[0], b = w[1];
    e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
    e[4] = b.x; e[5] = b.y; e[6] = b.z; e[7] = b.w;
  } else {
    unpack8(ld16(reinterpret_cast<const uint16_t*>(p.w) + 8 * vec), e);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] += p.w_bias;
}

// LayerNorm gamma and beta of one 16-byte column vector, read from global memory.
__device__ __forceinline__ void load_affine8(const FwdParams& p, int vec, float ga[8],
                                             float be[8]) {
  const float4* g = reinterpret_cast<const float4*>(p.w) + 2 * vec;
  const float4* b = reinterpret_cast<const float4*>(p.beta) + 2 * vec;
  const float4 g0 = g[0], g1 = g[1], b0 = b[0], b1 = b[1];
  ga[0] = g0.x; ga[1] = g0.y; ga[2] = g0.z; ga[3] = g0.w;
  ga[4] = g1.x; ga[5] = g1.y; ga[6] = g1.z; ga[7] = g1.w;
  be[0] = b0.x; be[1] = b0.y; be[2] = b0.z; be[3] = b0.w;
  be[4] = b1.x; be[5] = b1.y; be[6] = b1.z; be[7] = b1.w;
}

// The same through buffer descriptors: the row loop reads gamma and beta this way when
// they are not staged in LDS.  (Plain pointers here would let the compiler merge the LDS
// and global reads into generic flat loads, which wait on every outstanding row store.)
__device__ __forceinline__ void load_affine8_buf(rsrc_t g, rsrc_t b, int vec, float ga[8],
                                                 float be[8]) {
  const uint32_t off = (uint32_t)vec * 32u;
  const v4u g0 = bload16_keep(g, off), g1 = bload16_keep(g, off + 16);
  const v4u b0 = bload16_keep(b, off), b1 = bload16_keep(b, off + 16);
  ga[0] = __uint_as_float(g0.x); ga[1] = __uint_as_float(g0.y);
  ga[2] = __uint_as_float(g0.z); ga[3] = __uint_as_float(g0.w);
  ga[4] = __uint_as_float(g1.x); ga[5] = __uint_as_float(g1.y);
  ga[6] = __uint_as_float(g1.z); ga[7] = __uint_as_float(g1.w);
  be[0] = __uint_as_float(b0.x); be[1] = __uint_as_float(b0.y);
  be[2] = __uint_as_float(b0.z); be[3] = __uint_as_float(b0.w);
  be[4] = __uint_as_float(b1.x); be[5] = __uint_as_float(b1.y);
  be[6] = __uint_as_float(b1.z); be[7] = __uint_as_float(b1.w);
}

// Bytes of dynamic LDS a forward launch needs: `planes` FP32 planes of per-column
// parameters (0 when they are read from global memory) and double-buffered reduction
// slots of `stats` doubles per wave and row slot.
__host__ __device__ inline size_t fwd_lds_bytes(int nvec, int planes, int g, int wpr, int r,
                                                int stats) {
  return (size_t)16 * planes * nvec + (size_t)2 * g * wpr * r * stats * sizeof(double);
}

// The data one step of the forward loads: R row slots of VMAX vectors per tensor.
template <int R, int VMAX>
struct FwdStep {
  int64_t row[R];
  bool rok[R];
  v4u a[R][VMAX];                               // x, then h
  v4u b[R][VMAX];                               // residual
  v4u c[R][VMAX];                               // gate
  v4u ssc[R][VMAX], ssh[R][VMAX], sgt[R][VMAX]; // Ada style chunks
};

// Prefetching the next step (two steps in flight) is built in but off by default for the
// forward: on MI355X it measured slower for the forward rows (train forward at H=8192:
// 5.86 TB/s without, 5.67 TB/s with) -- HBM streams better with fewer bytes in flight per
// wave.  A tuning build enables it with DN_FWD_PREFETCH; it is used only when both steps
// fit in the VGPRs a wave may use at this block size.
constexpr bool fwd_double_buffer(int in, int epi, int vmax, int r, int nt) {
#ifndef DN_FWD_PREFETCH
  return false;
#endif
  const int tensors = 1 + (in != IN_PLAIN) + in_is_gated(in) +
                      3 * (epi == EPI_ADA_BF16 || epi == EPI_ADA_FP8) +
                      2 * (epi == EPI_LN_MOD_BF16) + (epi == EPI_SIGMOID_GATE);
  const int step = tensors * 4 * vmax * r;
  const int budget = nt >= 1024 ? 128 : 256;
  return 2 * step + 96 <= budget;
}

// The block's place in the row order.  With `xcd`, the blocks of each XCD are numbered
// consecutively (blocks are dealt to the 8 XCDs round-robin), so neighbouring rows stay on
// one XCD: the 1x128 block scales of neighbouring rows share 64-byte lines of their
// column-major array, which then fill in one XCD's L2 instead of leaving eight partial
// lines to be written back (measured on block FP8 [16384,7168]: bytes written 1.072 ->
// 1.000 of the algorithmic writes, +1.8 %).  Other forwards write no such side array and
// keep the plain order (tuning builds set DN_XCD_ROWS to order them all).
template <bool xcd>
__device__ __forceinline__ int row_block(int b, int n) {
#ifdef DN_XCD_ROWS
  constexpr bool on = true;
#else
  constexpr bool on = xcd;
#endif
  if (on && (n & 7) == 0) return (b & 7) * (n >> 3) + (b >> 3);
  return b;
}

template <int IN, int EPI, int TPR, int VMAX, int R, int NT>
__global__ void __launch_bounds__(NT) fwd_kernel(const FwdParams p) {
  extern __shared__ __align__(16) unsigned char dn_lds[];
  using Geom = RowGeom<TPR, R, NT>;
  using Step = FwdStep<R, VMAX>;
  constexpr int G = Geom::G;
  constexpr int WPR = Geom::WPR;
  constexpr int RPW = Geom::RPW;
  constexpr int RW = TPR < 64 ? TPR : 64;        // lanes of a row inside one wave
  constexpr bool kAda = (EPI == EPI_ADA_BF16 || EPI == EPI_ADA_FP8);
  constexpr bool kLN = epi_is_ln(EPI);
  constexpr bool kMod = (EPI == EPI_LN_MOD_BF16);
  constexpr bool kGatedIn = in_is_gated(IN);
  constexpr bool kSigGate = (EPI == EPI_SIGMOID_GATE);
  constexpr bool kLoadGate = kGatedIn || kSigGate;
  constexpr int kPlanes = fwd_weight_planes(EPI);
  constexpr int kStats = fwd_stats(EPI);
  constexpr bool kSilu = epi_is_silu(EPI);
  constexpr bool kStaticFp8 = (EPI == EPI_FP8 || EPI == EPI_ADA_FP8 || EPI == EPI_LN_FP8 ||
                               EPI == EPI_SILU_FP8);
  constexpr bool kFp8Out = (EPI == EPI_FP8 || EPI == EPI_FP8_BLOCK || EPI == EPI_ADA_FP8 ||
                            EPI == EPI_LN_FP8 || EPI == EPI_SILU_FP8);
  constexpr bool kDB = fwd_double_buffer(IN, EPI, VMAX, R, NT);
  // Rows are held packed (BF16 pairs) across the reduction and unpacked again for the
  // epilogue, halving their register footprint, except where the unpacked row fits
  // comfortably: a single input of at most four vectors per lane and row.
  constexpr bool kPackAcross = !(IN == IN_PLAIN && !kAda && !kMod && VMAX * R <= 4);

  const Geom geo;
  const int tid = threadIdx.x;
  const int lane = geo.lane;
  const int nvec = p.nvec;
  const uint32_t row_bf16 = 2u * (uint32_t)p.hidden;   // bytes of a BF16 row
  const uint32_t row_fp8 = (uint32_t)p.hidden;         // bytes of an FP8 row
  // Sub-wave rows: lanes past the row's last vector take an out-of-range offset.
  const bool lane_ok = TPR >= 64 || lane < nvec;
  float4* wl = reinterpret_cast<float4*>(dn_lds);
  float inv_scale = 1.0f;
  if constexpr (kStaticFp8) inv_scale = 1.0f / *p.scale;
  // SiLU's denominator factor: log2(e), times the static scale for FP8 outputs.
  float silu_c = kLog2E;
  if constexpr (EPI == EPI_SILU_FP8) silu_c = kLog2E * *p.scale;
  // SiLU + FP8: where every |z| of a vector in the wave is at most this limit, no output
  // needs the e4m3 clamp.  For z >= 0 the output is at most z / silu_c <= 440 (< 448, a few
  // ulps of rounding aside); for z < 0 its magnitude is at most (1/e) / scale, below 440
  // once silu_c >= 2e-3.  Any other scale (tiny, negative, NaN, infinite) disables it.
  float silu_lim = -1.0f;
  if constexpr (EPI == EPI_SILU_FP8)
    if (silu_c >= 2e-3f && silu_c <= 1e30f) silu_lim = 440.0f * silu_c;
  // Static FP8 without a modulation: the reciprocal scale is folded into the staged
  // per-column parameters (w_eff / scale; gamma / scale and beta / scale), one multiply
  // per element fewer in the epilogue.
  constexpr bool kFold = (EPI == EPI_FP8 || EPI == EPI_LN_FP8);
  double* red = reinterpret_cast<double*>(dn_lds + (p.w_in_lds ? (size_t)16 * kPlanes * nvec : 0));

  // FP8 outputs skip the NaN bypass of the e4m3 clamp on steps where no NaN can arise:
  // staged parameters of magnitude at most 2^100 (finite, and no overflow when a normalised
  // value, at most sqrt(hidden) in magnitude, is scaled by them), a finite 1/scale,
  // eps >= 0, and for every row of the wave a finite, nonzero rstd (which implies finite
  // inputs; LayerNorm also needs a finite mean).  Otherwise the NaN-safe clamp runs.
  bool params_ok = false;

  // Per-block set-up (staged per-column parameters, block-scale padding).  It runs after
  // the first step's row loads are issued, so the parameter fetch overlaps their latency.
  auto stage = [&]() {
    if (kPlanes > 0 && p.w_in_lds) {
      int nonfinite = 0;
      for (int i = tid; i < nvec; i += NT) {
        if constexpr (kLN) {
          float ga[8], be[8];
          load_affine8(p, i, ga, be);
          if constexpr (kFold) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              ga[k] *= inv_scale;
              be[k] *= inv_scale;
            }
          }
          if constexpr (kFp8Out) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
              nonfinite |= !(fabsf(ga[k]) <= 0x1p100f) | !(fabsf(be[k]) <= 0x1p100f);
          }
          wl[i] = make_float4(ga[0], ga[1], ga[2], ga[3]);
          wl[nvec + i] = make_float4(ga[4], ga[5], ga[6], ga[7]);
          wl[2 * nvec + i] = make_float4(be[0], be[1], be[2], be[3]);
          wl[3 * nvec + i] = make_float4(be[4], be[5], be[6], be[7]);
        } else {
          float e[8];
          load_weff8(p, i, e);
          if constexpr (kFold) {
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] *= inv_scale;
          }
          if constexpr (kSilu) {
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] *= kLog2E;   // see the SiLU epilogue
          }
          if constexpr (kFp8Out) {
#pragma unroll
            for (int k = 0; k < 8; ++k) nonfinite |= !(fabsf(e[k]) <= 0x1p100f);
          }
          wl[i] = make_float4(e[0], e[1], e[2], e[3]);
          wl[nvec + i] = make_float4(e[4], e[5], e[6], e[7]);
        }
      }
      if constexpr (kFp8Out) {
        params_ok = __syncthreads_or(nonfinite) == 0 && __builtin_isfinite(inv_scale) &&
                    p.eps >= 0.0f;
      } else {
        __syncthreads();
      }
    }

    if constexpr (EPI == EPI_FP8_BLOCK) {
      // Pad entries [rows, bld) of every block-scale column are written as zeros.
      const int64_t pad = p.bld - p.rows;
      if (blockIdx.x == 0 && pad > 0) {
        const int nb = p.hidden / 128;
        for (int64_t i = tid; i < (int64_t)nb * pad; i += NT)
          p.bscale[(i / pad) * p.bld + p.rows + (i % pad)] = 0.0f;
      }
    }
  };

  const double inv_hidden = 1.0 / (double)p.hidden;
  const double eps = (double)p.eps;
  int parity = 0;

  // 1) Issue every load of the step starting at row `base`.
  auto load = [&](Step& st, int64_t base) {
    const int64_t first = geo.first(base);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      st.row[rr] = geo.row(first, rr);
      st.rok[rr] = st.row[rr] < p.rows;
    }
    rsrc_t rx[R], rres[R], rg[R], rst[R], rsc[R], rsh[R];
    uint32_t ox[R], ores[R], og[R], ost[R], osc[R], osh[R];
    tensor_span<TPR, R, RPW>(p.x, p.sx, 2, 16, row_bf16, first, p.rows, lane, geo.j, lane_ok,
                             rx, ox);
    if constexpr (IN != IN_PLAIN)
      tensor_span<TPR, R, RPW>(p.r, p.sr, 2, 16, row_bf16, first, p.rows, lane, geo.j,
                               lane_ok, rres, ores);
    if constexpr (kLoadGate)
      tensor_span<TPR, R, RPW>(p.gate, p.sg, 2, 16, row_bf16, first, p.rows, lane, geo.j,
                               lane_ok, rg, og);
    if constexpr (kMod) {
      tensor_span<TPR, R, RPW>(p.msc, p.smsc, 2, 16, row_bf16, first, p.rows, lane, geo.j,
                               lane_ok, rsc, osc);
      tensor_span<TPR, R, RPW>(p.msh, p.smsh, 2, 16, row_bf16, first, p.rows, lane, geo.j,
                               lane_ok, rsh, osh);
    }
    if constexpr (kAda) {
      if (p.style_bcast) {
        // Every row reads the single style row.
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          rst[rr] = make_rsrc(p.style, 3u * row_bf16);
          ost[rr] = lane_ok ? (uint32_t)(lane * 16) : kOutOfRange;
        }
      } else {
        tensor_span<TPR, R, RPW>(p.style, p.sst, 2, 16, 3u * row_bf16, first, p.rows, lane,
                                 geo.j, lane_ok, rst, ost);
      }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        const uint32_t dv = (uint32_t)(v * TPR * 16);
        st.a[rr][v] = bload16(rx[rr], ox[rr] + dv);
        if constexpr (IN != IN_PLAIN) st.b[rr][v] = bload16(rres[rr], ores[rr] + dv);
        if constexpr (kLoadGate) st.c[rr][v] = bload16(rg[rr], og[rr] + dv);
        if constexpr (kMod) {
          st.ssc[rr][v] = bload16(rsc[rr], osc[rr] + dv);
          st.ssh[rr][v] = bload16(rsh[rr], osh[rr] + dv);
        }
        if constexpr (kAda) {
          if (p.style_bcast) {     // one style row serves every token: keep it cached
            st.ssc[rr][v] = bload16_keep(rst[rr], ost[rr] + dv);
            st.ssh[rr][v] = bload16_keep(rst[rr], ost[rr] + dv + row_bf16);
            st.sgt[rr][v] = bload16_keep(rst[rr], ost[rr] + dv + 2u * row_bf16);
          } else {
            st.ssc[rr][v] = bload16(rst[rr], ost[rr] + dv);
            st.ssh[rr][v] = bload16(rst[rr], ost[rr] + dv + row_bf16);
            st.sgt[rr][v] = bload16(rst[rr], ost[rr] + dv + 2u * row_bf16);
          }
        }
      }
    }
  };

  auto process = [&](Step& st, int64_t base) {
    const int64_t first = geo.first(base);
    // 2) h (rounded to BF16, stored early) and per-lane sums of squares of that BF16 h.
    double ss[R], s1[R];
    const bool tiny_eps = p.eps < 0x1p-80f;   // sums of squares in FP64 (sumsq8_d)
    {
      rsrc_t rh[R];
      uint32_t oh[R];
      if constexpr (IN != IN_PLAIN)
        tensor_span<TPR, R, RPW>(p.h, p.sh, 2, 16, p.h ? row_bf16 : 0u, first,
                                 p.h ? p.rows : first, lane, geo.j, lane_ok, rh, oh);
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        ss[rr] = 0.0;
        s1[rr] = 0.0;
#pragma unroll
        for (int v = 0; v < VMAX; ++v) {
          float fh[8];
          unpack8(st.a[rr][v], fh);
          if constexpr (IN == IN_ADD) {
            float fr[8];
            unpack8(st.b[rr][v], fr);
#pragma unroll
            for (int k = 0; k < 8; ++k) fh[k] = fh[k] + fr[k];
          } else if constexpr (IN == IN_GATED) {
            float fr[8], fg[8];
            unpack8(st.b[rr][v], fr);
            unpack8(st.c[rr][v], fg);
#pragma unroll
            for (int k = 0; k < 8; ++k) fh[k] = fmaf(fh[k], fg[k], fr[k]);
          } else if constexpr (IN == IN_GATED_BIAS) {
            float fr[8], fg[8];
            unpack8(st.b[rr][v], fr);
            unpack8(st.c[rr][v], fg);
#pragma unroll
            for (int k = 0; k < 8; ++k) fh[k] = fmaf(fh[k], fg[k] + p.gate_bias, fr[k]);
          }
          if constexpr (IN != IN_PLAIN) {
            st.a[rr][v] = pack8(fh);
            unpack8(st.a[rr][v], fh);       // the norm sees the BF16 h_new
            bstore16(rh[rr], oh[rr] + (uint32_t)(v * TPR * 16), st.a[rr][v]);
          }
          // Lanes past the row end loaded zeros: they add nothing.
          if constexpr (kLN) {
            // Exact FP64 terms: the sum and the sum of squares of a BF16 row carry no
            // rounding worth the name, so the one-pass variance stays accurate.
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const double d = (double)fh[k];
              s1[rr] += d;
              ss[rr] = fma(d, d, ss[rr]);
            }
          } else {
            ss[rr] += sumsq8_d(fh, tiny_eps);
          }
        }
      }
    }
    // 3) Row sums: DPP / row-swap steps inside the wave, then (rows over several waves)
    //    through LDS.
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        if constexpr (kPackAcross) keep_packed(st.a[rr][v]);
      }
      ss[rr] = group_sum<RW>(ss[rr]);
      if constexpr (kLN) s1[rr] = group_sum<RW>(s1[rr]);
    }
    if constexpr (WPR > 1) {
      const int wave_in_row = lane >> 6;
      double* slot = red + ((size_t)parity * G * WPR * R + (size_t)geo.grp * WPR * R) * kStats;
      if ((lane & 63) == 0) {
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
          slot[(wave_in_row * R + rr) * kStats] = ss[rr];
          if constexpr (kLN) slot[(wave_in_row * R + rr) * kStats + 1] = s1[rr];
        }
      }
      __syncthreads();
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        double s = 0.0, t = 0.0;
#pragma unroll
        for (int w8 = 0; w8 < WPR; ++w8) {
          s += slot[(w8 * R + rr) * kStats];
          if constexpr (kLN) t += slot[(w8 * R + rr) * kStats + 1];
        }
        ss[rr] = s;
        s1[rr] = t;
      }
      parity ^= 1;
    }

    // 4) RMSNorm: rstd = 1/sqrt(mean square + eps).  LayerNorm: mean = sum/H, variance =
    //    (sum of squares)/H - mean^2 (population variance), rstd = 1/sqrt(var + eps).
    //    FP64 throughout (rsqrt_f64: within 2^-52), one FP32 rounding of each result.  The
    //    LayerNorm mean is kept as an FP32 pair, mu = FP32(mean) and the rest (mean - mu)
    //    carried through the FMA that scales by rstd: (h - mean) * rstd is then formed within
    //    two FP32 roundings of its own value rather than of |mean|, so rows far from zero
    //    keep their centred values (and outputs near zero) to FP32 accuracy.
    float rs[R], mu[R], mu_lo[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      double r64;
      if constexpr (kLN) {
        const double mean = s1[rr] / (double)p.hidden;
        double var = ss[rr] / (double)p.hidden - mean * mean;
        var = var < 0.0 ? 0.0 : var;   // rounding can leave -0.x ulp; NaN stays NaN
        r64 = rsqrt_f64(var + eps);
        mu[rr] = (float)mean;
        // The rest of the mean, times -rstd: n = FMA(h - mu, rstd, mu_lo).  NaN when the mean
        // or rstd is not finite, as n is then.
        mu_lo[rr] = (float)(-(mean - (double)mu[rr]) * (double)(float)r64);
      } else {
        r64 = rsqrt_f64(ss[rr] * inv_hidden + eps);
        mu[rr] = 0.0f;
        mu_lo[rr] = 0.0f;
      }
      rs[rr] = (float)r64;
      if (p.rstd && lane == 0 && st.rok[rr]) p.rstd[st.row[rr]] = rs[rr];
    }
    bool fp8_fast = false;
    if constexpr (kFp8Out) {
      bool rows_ok = params_ok;
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
        rows_ok = rows_ok && __builtin_isfinite(rs[rr]) && rs[rr] > 0.0f &&
                  (!kLN || __builtin_isfinite(mu[rr]));
      fp8_fast = __builtin_amdgcn_ballot_w64(!rows_ok) == 0;
    }

    // 5) Epilogue: y = (h * r) * w_eff in FP32, then the output format.
    rsrc_t ry[R], rq[R], rgo[R];
    uint32_t oy[R], oq[R], ogo[R];
    if constexpr (EPI == EPI_BF16 || EPI == EPI_ADA_BF16 || EPI == EPI_FP8_BLOCK ||
                  EPI == EPI_LN_BF16 || EPI == EPI_LN_MOD_BF16 || EPI == EPI_SILU_BF16 ||
                  EPI == EPI_SIGMOID_GATE)
      tensor_span<TPR, R, RPW>(p.y, p.sy, 2, 16, p.y ? row_bf16 : 0u, first,
                               p.y ? p.rows : first, lane, geo.j, lane_ok, ry, oy);
    if constexpr (kFp8Out)
      tensor_span<TPR, R, RPW>(p.q, p.sq, 1, 8, row_fp8, first, p.rows, lane, geo.j, lane_ok,
                               rq, oq);
    if constexpr (kAda)
      tensor_span<TPR, R, RPW>(p.gate_out, p.sgo, 2, 16, p.gate_out ? row_bf16 : 0u, first,
                               p.gate_out ? p.rows : first, lane, geo.j, lane_ok, rgo, ogo);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        // Keep the scheduler from hoisting every vector's weight reads to the top.
        __builtin_amdgcn_sched_barrier(0);
        const int idx = v * TPR + lane;
        int widx = idx < nvec ? idx : nvec - 1;   // ragged lanes read a valid weight
        // The per-column parameters are the same for every row, so the compiler would keep
        // them in VGPRs across the row loop.  LayerNorm's gamma and beta take 8 VGPRs per
        // vector: 1024-thread blocks (128 VGPRs a lane) re-read them from LDS instead.
        constexpr bool kReread = kLN && NT >= 1024;
        if constexpr (kReread) asm volatile("" : "+v"(widx));
        const uint32_t d16 = (uint32_t)(v * TPR * 16);
        const uint32_t d8 = (uint32_t)(v * TPR * 8);
        float fh[8], we[8], yv[8];
        float silu_amax = 0.0f;   // largest |z| of the vector (SiLU)
        unpack8(st.a[rr][v], fh);
        if constexpr (kLN) {
          // n = FMA(h - mu, rstd, mu_lo) in FP32, then one FMA with gamma and beta (or with the
          // modulation's 1 + scale + scale_bias and shift + shift_bias).
          float nv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) nv[k] = fmaf(fh[k] - mu[rr], rs[rr], mu_lo[rr]);
          if constexpr (kMod) {
            float fsc[8], fsh[8];
            unpack8(st.ssc[rr][v], fsc);
            unpack8(st.ssh[rr][v], fsh);
#pragma unroll
            for (int k = 0; k < 8; ++k)
              yv[k] = fmaf(nv[k], (1.0f + fsc[k]) + p.scale_bias, fsh[k] + p.shift_bias);
          } else {
            float be[8];
            if (p.w_in_lds) {
              const float4 g0 = wl[widx], g1 = wl[nvec + widx];
              const float4 b0 = wl[2 * nvec + widx], b1 = wl[3 * nvec + widx];
              we[0] = g0.x; we[1] = g0.y; we[2] = g0.z; we[3] = g0.w;
              we[4] = g1.x; we[5] = g1.y; we[6] = g1.z; we[7] = g1.w;
              be[0] = b0.x; be[1] = b0.y; be[2] = b0.z; be[3] = b0.w;
              be[4] = b1.x; be[5] = b1.y; be[6] = b1.z; be[7] = b1.w;
            } else {
              load_affine8_buf(make_rsrc(p.w, 4u * (uint32_t)p.hidden),
                               make_rsrc(p.beta, 4u * (uint32_t)p.hidden), widx, we, be);
              if constexpr (kFold) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                  we[k] *= inv_scale;
                  be[k] *= inv_scale;
                }
              }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) yv[k] = fmaf(nv[k], we[k], be[k]);
          }
        } else {
          if (p.w_in_lds) {
            const float4 lo = wl[widx], hi = wl[nvec + widx];
            we[0] = lo.x; we[1] = lo.y; we[2] = lo.z; we[3] = lo.w;
            we[4] = hi.x; we[5] = hi.y; we[6] = hi.z; we[7] = hi.w;
          } else {
            load_weff8(p, widx, we);
            if constexpr (kFold) {
#pragma unroll
              for (int k = 0; k < 8; ++k) we[k] *= inv_scale;
            }
            if constexpr (kSilu) {
#pragma unroll
              for (int k = 0; k < 8; ++k) we[k] *= kLog2E;
            }
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) yv[k] = (fh[k] * rs[rr]) * we[k];
        }
        if constexpr (kSilu) {
          // SiLU(y) = y / (1 + e^-y).  The staged weights carry log2(e), so yv holds
          // z = y log2(e): e = 2^-|z| = e^-|y| on the hardware exp2 (v_exp_f32, its -|z|
          // argument an input modifier; < 0.75 ulp on normal results, measured), and
          //   SiLU(y) = max(z, z e) / (log2(e) (1 + e))
          // (z e > z exactly when z < 0, so the max picks y e^y / (1 + e^-|y|) for y < 0 and
          // y / (1 + e^-y) otherwise), the denominator one FMA and the hardware reciprocal
          // (v_rcp_f32, < 0.9 ulp).  For FP8 outputs the static scale joins the denominator.
          // Together within (|y| + 5) FP32 ulps of SiLU(y).  v_exp_f32 flushes results below
          // 2^-126 to zero, so rows with |y| > 80 take the accurate library exponential.
          float e[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float az = fabsf(yv[k]);
            silu_amax = fmaxf(silu_amax, az);
            e[k] = __builtin_amdgcn_exp2f(-az);
          }
          if (silu_amax > 80.0f * kLog2E) {
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] = expf(-fabsf(yv[k]) * kLn2);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k)
            yv[k] = max_of_results(yv[k], yv[k] * e[k]) *
                    __builtin_amdgcn_rcpf(fmaf(e[k], silu_c, silu_c));
        }

        if constexpr (kSigGate) {
          // y * sigmoid(g), sigmoid(g) = (1 or e) / (1 + e) with e = exp(-|g|), on the
          // hardware exp2 and reciprocal as in the SiLU epilogue (library exp for |g| > 80).
          float fg[8], e[8];
          unpack8(st.c[rr][v], fg);
          float amax = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float ag = fabsf(fg[k]);
            amax = fmaxf(amax, ag);
            e[k] = __builtin_amdgcn_exp2f(-ag * kLog2E);
          }
          if (amax > 80.0f) {
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] = expf(-fabsf(fg[k]));
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float sg = (fg[k] >= 0.0f ? 1.0f : e[k]) * __builtin_amdgcn_rcpf(1.0f + e[k]);
            yv[k] *= sg;
          }
        }

        if constexpr (EPI == EPI_BF16 || EPI == EPI_LN_BF16 || EPI == EPI_LN_MOD_BF16 ||
                      EPI == EPI_SILU_BF16 || EPI == EPI_SIGMOID_GATE) {
          bstore16(ry[rr], oy[rr] + d16, pack8(yv));
        } else if constexpr (EPI == EPI_FP8 || EPI == EPI_LN_FP8 || EPI == EPI_SILU_FP8) {
          if constexpr (!kFold && !kSilu) {
#pragma unroll
            for (int k = 0; k < 8; ++k) yv[k] *= inv_scale;
          }
          // SiLU vectors whose outputs all lie within the e4m3 range (a wave vote on the
          // bound above) convert without the clamp; a NaN, which the running maximum skips,
          // converts to the NaN code on either path.
          bool in_range = false;
          if constexpr (kSilu)
            in_range = __builtin_amdgcn_ballot_w64(!(silu_amax <= silu_lim)) == 0;
          if (in_range)
            bstore8(rq[rr], oq[rr] + d8, pack_fp8x8_in_range(yv));
          else if (fp8_fast)
            bstore8(rq[rr], oq[rr] + d8, pack_fp8x8<false>(yv));
          else
            bstore8(rq[rr], oq[rr] + d8, pack_fp8x8<true>(yv));
        } else if constexpr (EPI == EPI_FP8_BLOCK) {
          // The BF16 normalised value is both normed_out and the quantiser's input.
          const v4u nv = pack8(yv);
          bstore16(ry[rr], oy[rr] + d16, nv);
          float fn[8];
          unpack8(nv, fn);
          float amax = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(fn[k]));
          amax = row16_max(amax);               // one 1x128 block = 16 lanes x 8 values
          const float s = div_by_448(amax);     // FP32(amax / 448), correctly rounded
          // n / s as n * (1/s) on the hardware reciprocal (within 1 FP32 ulp).  Blocks with
          // a scale below 2^-100 (normalised values below ~1e-28) are scaled by 2^100 on
          // both sides first, so 1/s neither overflows nor leaves the normal range; a wave
          // vote leaves that multiply out when no lane's block needs it.
          const bool tiny = s < 0x1p-100f;
          const float sc = tiny ? 0x1p100f : 1.0f;
          const float rcp = s > 0.0f ? __builtin_amdgcn_rcpf(s * sc) : 0.0f;
          if (__builtin_amdgcn_ballot_w64(tiny) == 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) fn[k] = fn[k] * rcp;
          } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) fn[k] = (fn[k] * sc) * rcp;
          }
          // |n| <= amax and s is amax/448 correctly rounded, so |n * (1/s)| is at most
          // 448 * (1 + 2^-21) once every value is finite (the fast case: finite rows,
          // bounded weights): the conversion rounds it to at most 448 with no clamp (codes
          // overflow only from 464 up).  Otherwise the NaN-safe clamp runs.
          if (fp8_fast)
            bstore8(rq[rr], oq[rr] + d8, pack_fp8x8_in_range(fn));
          else
            bstore8(rq[rr], oq[rr] + d8, pack_fp8x8<true>(fn));
          if ((lane & 15) == 0 && st.rok[rr] && idx < nvec)
            p.bscale[(int64_t)(idx >> 4) * p.bld + st.row[rr]] = s;
        } else {  // AdaRMSNorm epilogue
          float fsc[8], fsh[8], o[8];
          unpack8(st.ssc[rr][v], fsc);
          unpack8(st.ssh[rr][v], fsh);
#pragma unroll
          for (int k = 0; k < 8; ++k) o[k] = fmaf(yv[k], 1.0f + fsc[k], fsh[k]);
          if constexpr (EPI == EPI_ADA_BF16) {
            bstore16(ry[rr], oy[rr] + d16, pack8(o));
          } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] *= inv_scale;
            bstore8(rq[rr], oq[rr] + d8, pack_fp8x8(o));
          }
          bstore16(rgo[rr], ogo[rr] + d16, st.sgt[rr][v]);
        }
      }
    }
  };

  const int64_t stride = (int64_t)gridDim.x * Geom::PER_ITER;
  if constexpr (kDB) {
    // Two steps in flight: the next step's loads are issued before the current step's
    // arithmetic, reduction and stores.
    Step s0, s1;
    int64_t base = (int64_t)row_block<EPI == EPI_FP8_BLOCK>(blockIdx.x, gridDim.x) *
                   Geom::PER_ITER;
    if (base < p.rows) load(s0, base);
    stage();
    while (base < p.rows) {
      int64_t nb = base + stride;
      if (nb < p.rows) load(s1, nb);
      process(s0, base);
      base = nb;
      if (base >= p.rows) break;
      nb = base + stride;
      if (nb < p.rows) load(s0, nb);
      process(s1, base);
      base = nb;
    }
  } else {
    // The first step is peeled so that its loads precede the set-up; the steady-state loop
    // keeps the load-then-process shape.
    Step s0;
    int64_t base = (int64_t)row_block<EPI == EPI_FP8_BLOCK>(blockIdx.x, gridDim.x) *
                   Geom::PER_ITER;
    if (base < p.rows) {
      load(s0, base);
      stage();
      process(s0, base);
      base += stride;
    } else {
      stage();
    }
    for (; base < p.rows; base += stride) {
      load(s0, base);
      process(s0, base);
    }
  }
}

// ---------------------------------------------------------------------------- row tiers
// (threads per row, 16-byte vectors per thread at most, rows per group per step, threads
//  per block).  The host takes the first tier, in this order, whose TPR*VMAX covers
//  hidden/8: up to 4 vectors per lane a row stays in one wave or less; wider rows spread
//  over more waves rather than holding more vectors per lane.  On MI355X fewer bytes in
//  flight per wave stream better (measured: train forward at H=8192 goes from 5.1 to
//  5.9 TB/s moving from 1 wave x 16 vectors to 4 waves x 4 vectors per row).  Between
//  the 4-vector tiers, a 3-vector tier of the same width takes rows of up to 3*TPR
//  vectors: no slot left empty, fewer registers, more waves resident (measured at H=3072,
//  5120, 6144, 10240 and 12288: +1-20 %, the most for plain RMSNorm and the Ada FP8 route,
//  none slower).  Two tiers of 5 and 7 waves fit the rows of 640 and 896 vectors exactly
//  (H = 5120, 7168), which a 256-lane tier fills to 83 and 88 %: the empty slots still
//  cost each wave its epilogue instructions, which weighs on the VALU-heavy 1x128 block FP8
//  (measured against the 256-lane tiers: block FP8 [22936,5120] +7.6 %, [16384,7168]
//  +5.5-5.9 %; the plain fused add -0.8 % and +1.4-2.2 %, within noise; 320 x 4 and
//  448 x 3 at H = 10240 and 448 x 4 at H = 14336 measured -5 to +3 %, not adopted).  The
//  tiers after the first sixteen are reachable only through dn_force_threads_per_row.
#define DN_FWD_TIERS(X)                                                         \
  X(0, 8, 1, 4, 256)    X(1, 16, 1, 4, 256)   X(2, 32, 1, 2, 256)              \
  X(3, 64, 1, 2, 256)   X(4, 64, 2, 1, 256)   X(5, 64, 3, 1, 256)              \
  X(6, 64, 4, 1, 256)   X(7, 128, 3, 1, 256)  X(8, 128, 4, 1, 256)             \
  X(9, 320, 2, 1, 320)  X(10, 256, 3, 1, 256) X(11, 448, 2, 1, 448)            \
  X(12, 256, 4, 1, 256) X(13, 512, 3, 1, 512) X(14, 512, 4, 1, 512)            \
  X(15, 1024, 4, 1, 1024)                                                      \
  X(16, 64, 6, 1, 256)  X(17, 64, 8, 1, 256)  X(18, 64, 12, 1, 256)            \
  X(19, 64, 16, 1, 256) X(20, 128, 7, 1, 256) X(21, 128, 8, 1, 256)            \
  X(22, 256, 8, 1, 256) X(23, 512, 8, 1, 512)

constexpr int kFwdTierCount = 24;
constexpr int kFwdAutoTiers = 16;   // tiers the automatic choice considers

// Largest VMAX an input/epilogue combination is built with: the Ada, gated and
// modulation routes keep five or six 16-byte vectors per column in flight, so they stop
// at 6.
constexpr int fwd_vmax_limit(int in, int epi) {
  return (in_is_gated(in) || epi == EPI_ADA_BF16 || epi == EPI_ADA_FP8 ||
          epi == EPI_LN_MOD_BF16 || epi == EPI_SIGMOID_GATE) ? 6 : 16;
}

}  // namespace dn
