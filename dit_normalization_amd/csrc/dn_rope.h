// Fused QK RMSNorm + 3-D rotary embedding + V copy for gfx950 (norm guide §5.2).
//
// One row is one token of the packed projection qkv = [Q heads | K heads | V heads], each
// head `hd` channels.  The row is read once; Q and K are each normalised across all of
// their heads (one rstd per token for Q and one for K), rotated pair by pair, and written
// to their own outputs; V is copied (or quantised) to its own output.
//
// Work units: interleaved pairs (2j, 2j+1) sit inside one 16-byte vector, so a unit is one
// vector (4 pairs).  NeoX pairs (j, j + hd/2) sit half a head apart, so a unit is the two
// vectors holding channels [8e, 8e+8) and [8e + hd/2, 8e + hd/2 + 8) of one head (8 pairs).
// A row's units are dealt to its TPR lanes round-robin (unit u to lane u mod TPR), so each
// load instruction of a wave reads consecutive vectors (interleaved) or consecutive
// half-head runs (NeoX).
//
// The rotation angles depend only on the token and the pair index j < hd/2, not on the
// head, so each step the row's lanes compute the token's hd/2 (cos, sin) pairs once and
// share them through LDS.  The angle is kept in revolutions: the position times an FP64
// inverse frequency over 2*pi, reduced to [-1/2, 1/2] by subtracting the nearest integer
// (exact in FP64), rounded once to FP32, and handed to the hardware sine and cosine
// (v_sin_f32 / v_cos_f32 take revolutions; measured within 1.3e-7 absolute over
// [-1/2, 1/2], as close as an FP32 library sincos of the rounded angle).  Two
// transcendental instructions per pair instead of a software sincos.  The
// inverse-frequency table itself (base^(-2i/count) per frame / height / width channel
// group, with the YaRN blend, divided by 2*pi) is built once per block.
#pragma once

#include "dn_device.h"

namespace dn {

struct RopeParams {
  const uint16_t* qkv;  int64_t sqkv;
  const void* wq;       const void* wk;  int w_f32;   // norm weights [nq*hd], [nk*hd]
  void* qo;             int64_t sqo;                  // outputs (BF16 or e4m3fn)
  void* ko;             int64_t sko;
  void* vo;             int64_t svo;
  const float* qk_scale;                              // FP8: device FP32 [1] for Q and K
  const float* v_scale;                               // FP8: device FP32 [1] for V
  int64_t rows;
  int nq, nk, nv, hd;
  int cf, ch, cw;                                     // channels per position group
  int ppf, pph, ppw;
  float eps, af;                                      // eps, attention factor
  double base, factor, low, high;                     // frequency table and YaRN blend
  int qk_norm;
  int w_in_lds;
  int nvec;                                           // 16-byte vectors per qkv row
  int nwvec;                                          // weight vectors: (nq + nk) * hd / 8
};

// Dynamic LDS of a launch: staged weights (two FP32 planes), the FP64 inverse-frequency
// table, double-buffered (cos, sin) tables for the G rows of a step, double-buffered
// cross-wave partial sums (two statistics).
__host__ __device__ inline size_t rope_weight_bytes(int w_in_lds, int nwvec) {
  return w_in_lds ? (size_t)32 * nwvec : 0;
}
__host__ __device__ inline size_t rope_lds_bytes(int w_in_lds, int nwvec, int hd, int g,
                                                 int wpr) {
  return rope_weight_bytes(w_in_lds, nwvec) + (size_t)8 * (hd / 2) +
         (size_t)2 * g * (hd / 2) * 8 + (size_t)2 * g * wpr * 2 * sizeof(double);
}

// Norm weight of one 16-byte column vector (index into the concatenated [Q | K] weights).
__device__ __forceinline__ void rope_weight8(const RopeParams& p, int vec, float e[8]) {
  const int qv = p.nq * p.hd / 8;
  const void* w = vec < qv ? p.wq : p.wk;
  const int i = vec < qv ? vec : vec - qv;
  if (p.w_f32) {
    const float4* f = reinterpret_cast<const float4*>(w) + 2 * i;
    const float4 a = f[0], b = f[1];
    e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
    e[4] = b.x; e[5] = b.y; e[6] = b.z; e[7] = b.w;
  } else {
    unpack8(ld16(reinterpret_cast<const uint16_t*>(w) + 8 * i), e);
  }
}

// 1/(2*pi), turning an angular frequency into revolutions per position.
constexpr double kInv2Pi = 0.15915494309189535;

// Waves per SIMD the register allocation must leave room for.  The kernel is latency-bound
// (vector ALUs and HBM both about half busy) and its occupancy is set by its VGPRs (2-3
// waves per SIMD unconstrained), so a tighter budget trades a few spills for more waves
// where that measured faster at the 3072-wide DiT layout: interleaved pairs with FP8
// outputs at 4 waves +7 %, NeoX pairs with BF16 outputs at 3 waves +3 %; the other two
// forms lost 7-16 % at 4 waves and gained nothing at 3.  Rows of 512 lanes or more keep
// the unconstrained budget (a 4-wave budget would spill up to 116 bytes per lane there).
template <int TPR, bool NEOX, bool FP8>
constexpr int rope_min_waves() {
  if (TPR > 256) return 1;
  return !NEOX && FP8 ? 4 : (NEOX && !FP8 ? 3 : 1);
}

// NeoX pairs with FP8 outputs: a unit's two 8-byte halves sit half a head apart, so a wave
// storing each half on its own covers only half of every 128-byte line (measured: 7.8 %
// more bytes written than the outputs hold).  Lanes 2k and 2k+1 hold units e and e + 1 of
// one head (e even; a head has an even number of units); they swap halves first, so the
// even lane stores the first halves of both units and the odd lane the second halves, 16
// consecutive bytes each, and the head's lanes write its lines whole in one store.
__device__ __forceinline__ void store_fp8_halves(rsrc_t r, uint32_t off, uint32_t half,
                                                 const v2u& a, const v2u& b, bool odd) {
  const v2u give = odd ? a : b;
  v2u take;
  take.x = dpp_u32<0xB1>(give.x);   // quad_perm [1, 0, 3, 2]: the pair partner's value
  take.y = dpp_u32<0xB1>(give.y);
  v4u out;
  if (odd) {
    out.x = take.x; out.y = take.y; out.z = b.x; out.w = b.y;
  } else {
    out.x = a.x; out.y = a.y; out.z = take.x; out.w = take.y;
  }
  bstore16(r, odd ? off + half - 8u : off, out);
}

template <int TPR, int VMAX, int NT, bool NEOX, bool FP8>
__global__ void __launch_bounds__(NT, (rope_min_waves<TPR, NEOX, FP8>()))
qkrope_kernel(const RopeParams p) {
  extern __shared__ __align__(16) unsigned char dn_lds[];
  using Geom = RowGeom<TPR, 1, NT>;
  constexpr int G = Geom::G;
  constexpr int WPR = Geom::WPR;
  constexpr int RPW = Geom::RPW;
  constexpr int RW = TPR < 64 ? TPR : 64;
  constexpr int VPU = NEOX ? 2 : 1;            // vectors per unit
  constexpr int UMAX = VMAX / VPU;             // units per lane
  static_assert(UMAX * VPU == VMAX, "VMAX must hold whole units");

  const Geom geo;
  const int tid = threadIdx.x;
  const int lane = geo.lane;
  const bool odd = (lane & 1) != 0;   // NeoX FP8 stores pair lanes 2k and 2k + 1
  const int hd = p.hd;
  const int half = hd / 2;
  const int vph = hd / 8;                      // vectors per head
  const int uph = vph / VPU;                   // units per head
  const int qk_heads = p.nq + p.nk;
  const int nunits = (qk_heads + p.nv) * uph;
  const uint32_t row_bf16 = (uint32_t)p.nvec * 16u;
  constexpr int OB = FP8 ? 8 : 16;             // output bytes per vector

  float4* wl = reinterpret_cast<float4*>(dn_lds);
  size_t off = rope_weight_bytes(p.w_in_lds, p.nwvec);
  double* freq = reinterpret_cast<double*>(dn_lds + off);
  off += (size_t)8 * half;
  float2* cs = reinterpret_cast<float2*>(dn_lds + off);
  off += (size_t)2 * G * half * 8;
  double* red = reinterpret_cast<double*>(dn_lds + off);

  // Per-block set-up: staged weights and the inverse-frequency table.
  if (p.qk_norm && p.w_in_lds) {
    for (int i = tid; i < p.nwvec; i += NT) {
      float e[8];
      rope_weight8(p, i, e);
      wl[i] = make_float4(e[0], e[1], e[2], e[3]);
      wl[p.nwvec + i] = make_float4(e[4], e[5], e[6], e[7]);
    }
  }
  for (int j = tid; j < half; j += NT) {
    int i, count;
    if (j < p.cf / 2) {
      i = j; count = p.cf;
    } else if (j < (p.cf + p.ch) / 2) {
      i = j - p.cf / 2; count = p.ch;
    } else {
      i = j - (p.cf + p.ch) / 2; count = p.cw;
    }
    double f = pow(p.base, -2.0 * (double)i / (double)count);
    if (p.factor != 1.0) {
      const double hi = p.high != p.low ? p.high : p.high + 0.001;
      double ramp = ((double)i - p.low) / (hi - p.low);
      ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
      f = f / p.factor * ramp + f * (1.0 - ramp);
    }
    freq[j] = f * kInv2Pi;    // revolutions per position
  }
  __syncthreads();

  float inv_qk = 1.0f, inv_v = 1.0f;
  if constexpr (FP8) {
    inv_qk = 1.0f / *p.qk_scale;
    inv_v = 1.0f / *p.v_scale;
  }
  // cos and sin carry the attention factor (and, for FP8 outputs, 1/scale).
  const float cs_mul = (float)((double)p.af * (double)inv_qk);
  // FP8 outputs skip the e4m3 clamp (and its NaN bypass) for a unit whose values a wave
  // vote shows in range.  A rotation keeps each pair's length, so a rotated value is at
  // most sqrt(2) max(|a|, |b|) |cs_mul| up to rounding: a Q or K unit whose inputs stay
  // within qk_lim gives values below 440.  V values only need |v / scale| <= 448, the
  // largest code (the conversion rounds to nearest and does not saturate).
  float qk_lim = -1.0f;
  if constexpr (FP8) {
    const float m = fabsf(cs_mul);
    if (m > 0.0f && m <= 1e30f) qk_lim = 440.0f / (1.4143f * m);
  }

  // This lane's units: byte offset of the first vector in the qkv row, class (0 Q, 1 K,
  // 2 V, 3 none), and the unit's index inside its head.
  uint32_t uoff[UMAX];
  int ucls[UMAX], uidx[UMAX], uvec[UMAX];
#pragma unroll
  for (int m = 0; m < UMAX; ++m) {
    const int u = lane + m * TPR;
    const int h = u / uph;
    const int e = u - h * uph;
    const int vec = h * vph + e;
    const bool ok = u < nunits;
    ucls[m] = !ok ? 3 : (h < p.nq ? 0 : (h < qk_heads ? 1 : 2));
    uidx[m] = e;
    uvec[m] = vec;
    uoff[m] = ok ? (uint32_t)vec * 16u : kOutOfRange;
  }

  // Token counts and patch grids stay below 2^31 (checked on the host): 32-bit index math.
  const uint32_t seq = (uint32_t)p.ppf * p.pph * p.ppw;
  const uint32_t hw = (uint32_t)p.pph * p.ppw;
  const double eps = (double)p.eps;
  int parity = 0;
  const int64_t stride = (int64_t)gridDim.x * Geom::PER_ITER;

  for (int64_t base = (int64_t)blockIdx.x * Geom::PER_ITER; base < p.rows; base += stride) {
    const int64_t first = geo.first(base);
    const int64_t row = geo.row(first, 0);

    // 1) Loads: the row's vectors of this lane's units.
    rsrc_t rx[1];
    uint32_t ox[1];
    tensor_span<TPR, 1, RPW>(p.qkv, p.sqkv, 2, 0, row_bf16, first, p.rows, lane, geo.j, true,
                             rx, ox);
    v4u va[UMAX], vb[UMAX];
#pragma unroll
    for (int m = 0; m < UMAX; ++m) {
      va[m] = bload16(rx[0], ox[0] + uoff[m]);
      if constexpr (NEOX) vb[m] = bload16(rx[0], ox[0] + uoff[m] + (uint32_t)uph * 16u);
    }

    // 2) The token's (cos, sin) table, computed by the row's lanes.
    {
      const uint32_t t = (uint32_t)row % seq;
      const double pf = (double)(t / hw);
      const double ph = (double)((t / (uint32_t)p.ppw) % (uint32_t)p.pph);
      const double pw = (double)(t % (uint32_t)p.ppw);
      float2* tab = cs + ((size_t)parity * G + geo.grp) * half;
      for (int j = lane; j < half; j += TPR) {
        const double pos = j < p.cf / 2 ? pf : (j < (p.cf + p.ch) / 2 ? ph : pw);
        const double rev = pos * freq[j];
        const float x = (float)(rev - rint(rev));       // in [-1/2, 1/2] revolutions
        tab[j] = make_float2(__builtin_amdgcn_cosf(x) * cs_mul,
                             __builtin_amdgcn_sinf(x) * cs_mul);
      }
    }

    // 3) Sums of squares of the Q and K channels.
    double sq = 0.0, sk = 0.0;
    const bool tiny_eps = p.eps < 0x1p-80f;   // sums of squares in FP64 (sumsq8_d)
#pragma unroll
    for (int m = 0; m < UMAX; ++m) {
      float f[8];
      unpack8(va[m], f);
      constexpr bool kJointVote = NEOX && !FP8;   // a measured scheduling preference
      double s = sumsq8_d<kJointVote>(f, tiny_eps);
      if constexpr (NEOX) {
        unpack8(vb[m], f);
        s += sumsq8_d<kJointVote>(f, tiny_eps);
      }
      sq += ucls[m] == 0 ? s : 0.0;
      sk += ucls[m] == 1 ? s : 0.0;
    }
    sq = group_sum<RW>(sq);
    sk = group_sum<RW>(sk);
    __syncthreads();   // the (cos, sin) table is complete; row partials may be shared
    if constexpr (WPR > 1) {
      const int wave_in_row = lane >> 6;
      double* slot = red + ((size_t)parity * G * WPR + (size_t)geo.grp * WPR) * 2;
      if ((lane & 63) == 0) {
        slot[wave_in_row * 2] = sq;
        slot[wave_in_row * 2 + 1] = sk;
      }
      __syncthreads();
      double a = 0.0, b = 0.0;
#pragma unroll
      for (int w8 = 0; w8 < WPR; ++w8) {
        a += slot[w8 * 2];
        b += slot[w8 * 2 + 1];
      }
      sq = a;
      sk = b;
    }
    float rq = 1.0f, rk = 1.0f;
    if (p.qk_norm) {
      rq = (float)rsqrt_f64(sq / (double)(p.nq * hd) + eps);
      rk = (float)rsqrt_f64(sk / (double)(p.nk * hd) + eps);
    }

    // 4) Epilogue: normalise, rotate, store to the unit's output.
    rsrc_t rqo[1], rko[1], rvo[1];
    uint32_t oqo[1], oko[1], ovo[1];
    tensor_span<TPR, 1, RPW>(p.qo, p.sqo, OB / 8, 0, (uint32_t)(p.nq * hd) * (OB / 8), first,
                             p.rows, lane, geo.j, true, rqo, oqo);
    tensor_span<TPR, 1, RPW>(p.ko, p.sko, OB / 8, 0, (uint32_t)(p.nk * hd) * (OB / 8), first,
                             p.rows, lane, geo.j, true, rko, oko);
    tensor_span<TPR, 1, RPW>(p.vo, p.svo, OB / 8, 0, (uint32_t)(p.nv * hd) * (OB / 8), first,
                             p.rows, lane, geo.j, true, rvo, ovo);
    const float2* tab = cs + ((size_t)parity * G + geo.grp) * half;
#pragma unroll
    for (int m = 0; m < UMAX; ++m) {
      __builtin_amdgcn_sched_barrier(0);
      const int cls = ucls[m];
      if (cls == 3) continue;
      if (cls == 2) {
        // V: a bit copy, or e4m3fn(v / v_scale).
        const uint32_t vo = (uint32_t)(uvec[m] - qk_heads * vph) * OB;
        if constexpr (FP8) {
          float f[8];
          unpack8(va[m], f);
#pragma unroll
          for (int k = 0; k < 8; ++k) f[k] *= inv_v;
          if constexpr (NEOX) {
            const v2u qa = pack_fp8x8_voted(f, 448.0f);
            unpack8(vb[m], f);
#pragma unroll
            for (int k = 0; k < 8; ++k) f[k] *= inv_v;
            const v2u qb = pack_fp8x8_voted(f, 448.0f);
            store_fp8_halves(rvo[0], ovo[0] + vo, (uint32_t)uph * OB, qa, qb, odd);
          } else {
            bstore8(rvo[0], ovo[0] + vo, pack_fp8x8_voted(f, 448.0f));
          }
        } else {
          bstore16(rvo[0], ovo[0] + vo, va[m]);
          if constexpr (NEOX) bstore16(rvo[0], ovo[0] + vo + (uint32_t)uph * OB, vb[m]);
        }
        continue;
      }
      const float r = cls == 0 ? rq : rk;
      float fa[8], fb[8];
      unpack8(va[m], fa);
      if constexpr (NEOX) unpack8(vb[m], fb);
      if (p.qk_norm) {
        float w[8];
        const int wv = uvec[m];
        if (p.w_in_lds) {
          const float4 lo = wl[wv], hi = wl[p.nwvec + wv];
          w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
          w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
        } else {
          rope_weight8(p, wv, w);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) fa[k] = (fa[k] * r) * w[k];
        if constexpr (NEOX) {
          const int wv2 = wv + uph;
          if (p.w_in_lds) {
            const float4 lo = wl[wv2], hi = wl[p.nwvec + wv2];
            w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
            w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
          } else {
            rope_weight8(p, wv2, w);
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) fb[k] = (fb[k] * r) * w[k];
        }
      }
      float oa[8], ob[8];
      if constexpr (NEOX) {
        // pairs (fa[k], fb[k]) = channels (8e + k, 8e + k + hd/2): pair index 8e + k
        const float4* t4 = reinterpret_cast<const float4*>(tab + 8 * uidx[m]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 c = t4[q];   // (cos, sin) of pairs 2q and 2q+1
          const float c0 = c.x, s0 = c.y, c1 = c.z, s1 = c.w;
          oa[2 * q] = fmaf(fa[2 * q], c0, -(fb[2 * q] * s0));
          ob[2 * q] = fmaf(fa[2 * q], s0, fb[2 * q] * c0);
          oa[2 * q + 1] = fmaf(fa[2 * q + 1], c1, -(fb[2 * q + 1] * s1));
          ob[2 * q + 1] = fmaf(fa[2 * q + 1], s1, fb[2 * q + 1] * c1);
        }
      } else {
        // pairs (fa[2q], fa[2q+1]) = channels (8e + 2q, 8e + 2q + 1): pair index 4e + q
        const float4* t4 = reinterpret_cast<const float4*>(tab + 4 * uidx[m]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float4 c = t4[q];
          const float a0 = fa[4 * q], b0 = fa[4 * q + 1], a1 = fa[4 * q + 2], b1 = fa[4 * q + 3];
          oa[4 * q] = fmaf(a0, c.x, -(b0 * c.y));
          oa[4 * q + 1] = fmaf(a0, c.y, b0 * c.x);
          oa[4 * q + 2] = fmaf(a1, c.z, -(b1 * c.w));
          oa[4 * q + 3] = fmaf(a1, c.w, b1 * c.z);
        }
      }
      bool in_range = false;
      if constexpr (FP8) {
        float am = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          am = fmaxf(am, fabsf(fa[k]));
          if constexpr (NEOX) am = fmaxf(am, fabsf(fb[k]));
        }
        in_range = __builtin_amdgcn_ballot_w64(!(am <= qk_lim)) == 0;
      }
      const int vbase = cls == 0 ? uvec[m] : uvec[m] - p.nq * vph;
      const uint32_t o = (uint32_t)vbase * OB;
      if (cls == 0) {
        if constexpr (FP8) {
          if constexpr (NEOX) {
            v2u qa, qb;
            if (in_range) {
              qa = pack_fp8x8_in_range(oa);
              qb = pack_fp8x8_in_range(ob);
            } else {
              qa = pack_fp8x8(oa);
              qb = pack_fp8x8(ob);
            }
            store_fp8_halves(rqo[0], oqo[0] + o, (uint32_t)uph * OB, qa, qb, odd);
          } else if (in_range) {
            bstore8(rqo[0], oqo[0] + o, pack_fp8x8_in_range(oa));
          } else {
            bstore8(rqo[0], oqo[0] + o, pack_fp8x8(oa));
          }
        } else {
          bstore16(rqo[0], oqo[0] + o, pack8(oa));
          if constexpr (NEOX) bstore16(rqo[0], oqo[0] + o + (uint32_t)uph * OB, pack8(ob));
        }
      } else {
        if constexpr (FP8) {
          if constexpr (NEOX) {
            v2u qa, qb;
            if (in_range) {
              qa = pack_fp8x8_in_range(oa);
              qb = pack_fp8x8_in_range(ob);
            } else {
              qa = pack_fp8x8(oa);
              qb = pack_fp8x8(ob);
            }
            store_fp8_halves(rko[0], oko[0] + o, (uint32_t)uph * OB, qa, qb, odd);
          } else if (in_range) {
            bstore8(rko[0], oko[0] + o, pack_fp8x8_in_range(oa));
          } else {
            bstore8(rko[0], oko[0] + o, pack_fp8x8(oa));
          }
        } else {
          bstore16(rko[0], oko[0] + o, pack8(oa));
          if constexpr (NEOX) bstore16(rko[0], oko[0] + o + (uint32_t)uph * OB, pack8(ob));
        }
      }
    }
    parity ^= 1;
  }
}

// Row tiers (threads per row, 16-byte vectors per lane, threads per block), tried in
// order: the first whose TPR * VMAX / (vectors per unit) covers the row's units is used.
#define DN_ROPE_TIERS(X)                                                            \
  X(0, 8, 2, 256)   X(1, 8, 4, 256)   X(2, 16, 4, 256)  X(3, 32, 4, 256)          \
  X(4, 64, 4, 256)  X(5, 64, 6, 256)  X(6, 128, 4, 256) X(7, 128, 6, 256)         \
  X(8, 256, 4, 256) X(9, 256, 6, 256) X(10, 512, 4, 512) X(11, 512, 6, 512)       \
  X(12, 1024, 4, 1024)

constexpr int kRopeTierCount = 13;

}  // namespace dn
