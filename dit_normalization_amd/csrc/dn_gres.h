// Gated-residual RMSNorm (and the next RMSNorm in the same launch) for gfx950.
//
// Per row: n = (branch * r_b) * w_eff (FP32, unrounded), h = FMA(gate, n, residual) rounded
// once to BF16 and stored over the residual; with NEXT, the BF16 stream h is normalised
// again in the same step (a second row reduction) and y = BF16((h * r_h) * w2_eff) is
// written.  The row machinery is the forward engine's: a row owned by TPR lanes, 16-byte
// buffer loads, FP64 sums of exact squares, LDS across the waves of a row, per-column
// weights staged in LDS, persistent blocks.
#pragma once

#include "dn_fwd.h"

namespace dn {

struct GresParams {
  const uint16_t* b;  int64_t sb;              // branch
  uint16_t* r;        int64_t sr;              // residual stream, overwritten with h
  const uint16_t* g;  int64_t sg;  int g_bcast;  // gate rows, or one row for every token
  const void* w;      int w_f32;   float w_bias;
  const void* w2;     int w2_f32;  float w2_bias;  // NEXT
  uint16_t* y;        int64_t sy;              // NEXT output
  int64_t rows;
  int hidden;
  int nvec;
  float eps;
  int w_in_lds;
};

__host__ __device__ inline size_t gres_lds_bytes(int nvec, int w_in_lds, bool next, int g,
                                                 int wpr, int r) {
  const int planes = w_in_lds ? (next ? 4 : 2) : 0;
  return (size_t)16 * planes * nvec + (size_t)(next ? 2 : 1) * 2 * g * wpr * r * sizeof(double);
}

__device__ __forceinline__ void gres_weight8(const void* w, int f32, float bias, int vec,
                                             float e[8]) {
  if (f32) {
    const float4* f = reinterpret_cast<const float4*>(w) + 2 * vec;
    const float4 a = f[0], c = f[1];
    e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
    e[4] = c.x; e[5] = c.y; e[6] = c.z; e[7] = c.w;
  } else {
    unpack8(ld16(reinterpret_cast<const uint16_t*>(w) + 8 * vec), e);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] += bias;
}

// Sum of a per-lane FP64 value over the row: group_sum in the wave, then LDS across the row's waves
// (slot set `s` of this step's parity).
template <int RW, int WPR, int R, int G>
__device__ __forceinline__ void gres_row_sum(double (&v)[R], double* slots, int parity,
                                             int grp, int lane) {
#pragma unroll
  for (int rr = 0; rr < R; ++rr) v[rr] = group_sum<RW>(v[rr]);
  if constexpr (WPR > 1) {
    double* slot = slots + (size_t)parity * G * WPR * R + (size_t)grp * WPR * R;
    if ((lane & 63) == 0) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) slot[(lane >> 6) * R + rr] = v[rr];
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      double s = 0.0;
#pragma unroll
      for (int w8 = 0; w8 < WPR; ++w8) s += slot[w8 * R + rr];
      v[rr] = s;
    }
  }
}

template <int TPR, int VMAX, int R, int NT, bool NEXT>
__global__ void __launch_bounds__(NT) gres_kernel(const GresParams p) {
  extern __shared__ __align__(16) unsigned char dn_lds[];
  using Geom = RowGeom<TPR, R, NT>;
  constexpr int G = Geom::G;
  constexpr int WPR = Geom::WPR;
  constexpr int RPW = Geom::RPW;
  constexpr int RW = TPR < 64 ? TPR : 64;
  const Geom geo;
  const int tid = threadIdx.x;
  const int lane = geo.lane;
  const int nvec = p.nvec;
  const uint32_t row_bf16 = 2u * (uint32_t)p.hidden;
  const bool lane_ok = TPR >= 64 || lane < nvec;
  constexpr int kPlanes = NEXT ? 4 : 2;
  float4* wl = reinterpret_cast<float4*>(dn_lds);
  double* red = reinterpret_cast<double*>(dn_lds + (p.w_in_lds ? (size_t)16 * kPlanes * nvec : 0));
  double* red2 = red + (size_t)2 * G * WPR * R;

  if (p.w_in_lds) {
    for (int i = tid; i < nvec; i += NT) {
      float e[8];
      gres_weight8(p.w, p.w_f32, p.w_bias, i, e);
      wl[i] = make_float4(e[0], e[1], e[2], e[3]);
      wl[nvec + i] = make_float4(e[4], e[5], e[6], e[7]);
      if constexpr (NEXT) {
        gres_weight8(p.w2, p.w2_f32, p.w2_bias, i, e);
        wl[2 * nvec + i] = make_float4(e[0], e[1], e[2], e[3]);
        wl[3 * nvec + i] = make_float4(e[4], e[5], e[6], e[7]);
      }
    }
    __syncthreads();
  }

  const double inv_hidden = 1.0 / (double)p.hidden;
  const double eps = (double)p.eps;
  int parity = 0;
  const int64_t stride = (int64_t)gridDim.x * Geom::PER_ITER;
  for (int64_t base = (int64_t)blockIdx.x * Geom::PER_ITER; base < p.rows; base += stride) {
    const int64_t first = geo.first(base);
    rsrc_t rb[R], rr_[R], rg[R];
    uint32_t ob[R], or_[R], og[R];
    tensor_span<TPR, R, RPW>(p.b, p.sb, 2, 16, row_bf16, first, p.rows, lane, geo.j, lane_ok,
                             rb, ob);
    tensor_span<TPR, R, RPW>(p.r, p.sr, 2, 16, row_bf16, first, p.rows, lane, geo.j, lane_ok,
                             rr_, or_);
    if (p.g_bcast) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        rg[rr] = make_rsrc(p.g, row_bf16);
        og[rr] = lane_ok ? (uint32_t)(lane * 16) : kOutOfRange;
      }
    } else {
      tensor_span<TPR, R, RPW>(p.g, p.sg, 2, 16, row_bf16, first, p.rows, lane, geo.j,
                               lane_ok, rg, og);
    }
    v4u vb[R][VMAX], vr[R][VMAX], vg[R][VMAX];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        const uint32_t dv = (uint32_t)(v * TPR * 16);
        vb[rr][v] = bload16(rb[rr], ob[rr] + dv);
        vr[rr][v] = bload16(rr_[rr], or_[rr] + dv);
        vg[rr][v] = p.g_bcast ? bload16_keep(rg[rr], og[rr] + dv) : bload16(rg[rr], og[rr] + dv);
      }
    }

    // rstd of the branch
    double ss[R];
    const bool tiny_eps = p.eps < 0x1p-80f;   // sums of squares in FP64 (sumsq8_d)
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      ss[rr] = 0.0;
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        float f[8];
        unpack8(vb[rr][v], f);
        ss[rr] += sumsq8_d(f, tiny_eps);
      }
#pragma unroll
      for (int v = 0; v < VMAX; ++v) keep_packed(vb[rr][v]);
    }
    gres_row_sum<RW, WPR, R, G>(ss, red, parity, geo.grp, lane);
    float rs[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) rs[rr] = (float)rsqrt_f64(ss[rr] * inv_hidden + eps);

    // h = BF16(FMA(gate, n, residual)), stored over the residual; kept for the next norm
    double s2[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      s2[rr] = 0.0;
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        __builtin_amdgcn_sched_barrier(0);
        const int idx = v * TPR + lane;
        const int widx = idx < nvec ? idx : nvec - 1;
        float fb[8], fr[8], fg[8], we[8], h[8];
        unpack8(vb[rr][v], fb);
        unpack8(vr[rr][v], fr);
        unpack8(vg[rr][v], fg);
        if (p.w_in_lds) {
          const float4 lo = wl[widx], hi = wl[nvec + widx];
          we[0] = lo.x; we[1] = lo.y; we[2] = lo.z; we[3] = lo.w;
          we[4] = hi.x; we[5] = hi.y; we[6] = hi.z; we[7] = hi.w;
        } else {
          gres_weight8(p.w, p.w_f32, p.w_bias, widx, we);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = fmaf(fg[k], (fb[k] * rs[rr]) * we[k], fr[k]);
        const v4u hp = pack8(h);
        bstore16(rr_[rr], or_[rr] + (uint32_t)(v * TPR * 16), hp);
        if constexpr (NEXT) {
          vb[rr][v] = hp;            // the BF16 stream, for the next norm
          float fh[8];
          unpack8(hp, fh);
          s2[rr] += sumsq8_d(fh, tiny_eps);
        }
      }
    }

    if constexpr (NEXT) {
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
#pragma unroll
        for (int v = 0; v < VMAX; ++v) keep_packed(vb[rr][v]);
      }
      gres_row_sum<RW, WPR, R, G>(s2, red2, parity, geo.grp, lane);
      rsrc_t ry[R];
      uint32_t oy[R];
      tensor_span<TPR, R, RPW>(p.y, p.sy, 2, 16, row_bf16, first, p.rows, lane, geo.j,
                               lane_ok, ry, oy);
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const float r2 = (float)rsqrt_f64(s2[rr] * inv_hidden + eps);
#pragma unroll
        for (int v = 0; v < VMAX; ++v) {
          __builtin_amdgcn_sched_barrier(0);
          const int idx = v * TPR + lane;
          const int widx = idx < nvec ? idx : nvec - 1;
          float fh[8], we[8], yv[8];
          unpack8(vb[rr][v], fh);
          if (p.w_in_lds) {
            const float4 lo = wl[2 * nvec + widx], hi = wl[3 * nvec + widx];
            we[0] = lo.x; we[1] = lo.y; we[2] = lo.z; we[3] = lo.w;
            we[4] = hi.x; we[5] = hi.y; we[6] = hi.z; we[7] = hi.w;
          } else {
            gres_weight8(p.w2, p.w2_f32, p.w2_bias, widx, we);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) yv[k] = (fh[k] * r2) * we[k];
          bstore16(ry[rr], oy[rr] + (uint32_t)(v * TPR * 16), pack8(yv));
        }
      }
    }
    parity ^= 1;
  }
}

}  // namespace dn
