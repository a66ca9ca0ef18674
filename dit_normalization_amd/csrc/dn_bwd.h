// Training backward of RMSNorm for gfx950: dx plus a bitwise-deterministic FP32 dw.
//
// Producers (one block per fixed chunk of rows): chunk c of C holds rows c, c + C, c + 2C,
// ... (C = min(rows, 256)), so at any moment the blocks stream neighbouring rows (HBM
// serves interleaved streams better than C separate contiguous ranges).  Every thread owns
// a fixed set of 16-byte column vectors for the whole chunk, so its slice of dw stays in
// FP64 registers while the block streams the chunk's rows:
//     per row t:  c_t  = (1/H) sum_j g*w_eff*x         (lane partials in FP32, then FP64)
//                 dx   = BF16(r*(g*w_eff - x*(r^2*c_t)) [+ g_residual])
//     per column: P[chunk][j] += (g*x) * r              (exact products, FP64 sums)
// A row is split over TPR threads (over several waves for wide rows, meeting in LDS); for
// narrow rows several row groups run side by side and their FP64 sums are added in group
// order at the end.  The chunk's FP64 column sums are written as one workspace row.
//
// Reduction: dw_j = FP32(sum over chunks of P[chunk][j]) in a fixed order -- the chunk
// rows are cut into eight contiguous ranges, each range is added in chunk order, then the
// eight range sums in range order.  The chunk table depends only on (rows, hidden), never
// on the device, so dw is bitwise reproducible on any MI355X.
//
// The reduction is a second launch.  The pages' design finishes it inside the first one
// (the block that completes last reduces the partials), which needs every block's chunk
// row visible to another block within the kernel.  On MI355X the eight XCDs' L2 caches
// are not coherent with one another, so that takes a release (an L2 write-back) in every
// producing block and an acquire (an L2 invalidation) in every reducing block.  Measured
// at [2048, 8192] and [16384, 8192], with blocks taking producer or reducer roles by a
// ticket: 56 / 165 us with one release per producing block and one acquire per reducing
// block (138 / 244 us with a release in every wave; 49 / 156 us with no release at all,
// which is unsafe), against 30.5 / 139 us for two launches, whose boundary does the same
// cache maintenance once.
#pragma once

#include "dn_device.h"

namespace dn {

// Fixed upper bound on the number of row chunks (the workspace holds this many rows of
// FP64 column sums).  chunks = min(rows, kMaxChunks).
constexpr int kMaxChunks = 256;
// The reduction: one block of 256 threads per 32 columns (so a hidden of 8192 keeps every
// CU of the chip busy), thread t adding chunk range t / 32 of column t % 32.  The chunk
// rows are cut into kReduceRanges contiguous ranges whose sums are added last, in range
// order.
constexpr int kReduceThreads = 256;
constexpr int kReduceRanges = 8;
constexpr int kReduceCols = kReduceThreads / kReduceRanges;

struct BwdParams {
  uint16_t* dx;          int64_t sdx;
  const uint16_t* g;     int64_t sg;
  const uint16_t* x;     int64_t sx;
  const uint16_t* gres;  int64_t sgr;    // nullable
  const void* w;         int w_f32;      float w_bias;
  const float* rstd;
  double* part;                          // [chunks][hidden]
  int64_t rows;
  int hidden;
  int nvec;
  int chunks;
};

// dw of the reduction block's 32 columns from the chunk rows: each thread adds one range of
// chunk rows of one column (all its loads issued before the first add), the ranges meet in
// LDS and are added in range order; one rounding to FP32 (then to BF16 when dw_bf16, as a
// BF16 weight's gradient is the FP32 value rounded once more).
template <int NT>
__global__ void __launch_bounds__(NT) bwd_reduce_kernel(void* dw, int dw_bf16, const double* part,
                                                        int hidden, int chunks) {
  static_assert(NT == kReduceThreads, "one thread per (range, column)");
  constexpr int kMaxLen = kMaxChunks / kReduceRanges;
  __shared__ double red[kReduceRanges][kReduceCols];
  const int c_local = threadIdx.x % kReduceCols;
  const int range = threadIdx.x / kReduceCols;
  const int col = blockIdx.x * kReduceCols + c_local;
  const int cb = range * chunks / kReduceRanges, ce = (range + 1) * chunks / kReduceRanges;
  const int len = ce - cb;
  // Every load is issued unconditionally, at an index clamped into the chunk rows (no branch
  // between a load and the next, so all of them are in flight before the first add); the
  // range's own values are then added in chunk order and the others dropped by a select
  // (adding +0.0 to a sum that started at +0.0 changes no bit).
  const int cc = col < hidden ? col : hidden - 1;
  double v[kMaxLen];
#pragma unroll
  for (int i = 0; i < kMaxLen; ++i) {
    const int c = cb + i < chunks ? cb + i : chunks - 1;
    v[i] = part[(int64_t)c * hidden + cc];
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxLen; ++i) s += i < len ? v[i] : 0.0;
  red[range][c_local] = s;
  __syncthreads();
  if ((int)threadIdx.x < kReduceCols && col < hidden) {
    double t = 0.0;
#pragma unroll
    for (int r = 0; r < kReduceRanges; ++r) t += red[r][threadIdx.x];
    const float f = (float)t;
    if (dw_bf16)
      static_cast<uint16_t*>(dw)[col] = (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
    else
      static_cast<float*>(dw)[col] = f;
  }
}

__device__ __forceinline__ void bwd_weff8(const BwdParams& p, int vec, float e[8]) {
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

// The row groups' column sums meet in LDS with a pitch of 9 doubles per 16-byte column
// vector: a wave writing one sum of 64 consecutive vectors then touches every bank once
// (72-byte lane stride), and consecutive threads reading consecutive columns read
// consecutive doubles.
constexpr int kCombPitch = 9;

// Cache policy of the chunk-row stores: device scope (sc1), so the rows are written through
// to memory as they are stored rather than left dirty in the XCD's L2 for the kernel's end
// to write back; not non-temporal, which kept them from the cache the reduction reads
// through.  Measured against the default policy: [2048, 8192] +2.9 %, [4096, 8192] +2.7 %,
// [16384, 8192] +1.2 % (80 interleaved launches); non-temporal as well -4 % and -1 %.
constexpr int kChunkStorePolicy = 16;

// Dynamic LDS of a producer launch: the double-buffered dot-product slots, and the row
// groups' column sums when they meet at the end.
__host__ __device__ inline size_t bwd_lds_bytes(int g, int wpr, int rb, int nt, int vb) {
  const size_t red = (size_t)2 * g * wpr * rb * sizeof(double);
  const size_t comb = g > 1 ? (size_t)nt * vb * kCombPitch * sizeof(double) : 0;
  return red > comb ? red : comb;
}

// One step of stage 1: the RB row slots of this thread's row group and their data.
template <int VB, int RB>
struct BwdStep {
  int64_t row[RB];
  bool rok[RB];
  float rs[RB];
  v4u g[RB][VB], x[RB][VB], r[RB][VB];
};

// Two steps are kept in flight when both fit in the VGPRs a wave may use at this block size
// (the data of a step, the FP64 column sums, the weights and ~64 working registers): a
// block owns a whole CU here, so without the prefetch its memory pipe would idle through
// every cross-wave barrier (measured 5.29 -> 5.42 TB/s for stage 1 at [16384, 8192]).
constexpr bool bwd_double_buffer(int vb, int rb, int nt, bool gres) {
#ifdef DN_NO_PREFETCH
  return false;
#endif
  const int step = rb * vb * 4 * (gres ? 3 : 2);
  const int budget = nt >= 1024 ? 128 : 256;
  return 2 * step + vb * 16 + vb * 8 + 64 <= budget;
}

template <int TPR, int VB, int RB, int NT, bool GRES>
__global__ void __launch_bounds__(NT) bwd_partials_kernel(const BwdParams p) {
  constexpr bool kDB = bwd_double_buffer(VB, RB, NT, GRES);
  extern __shared__ __align__(16) unsigned char dn_lds[];
  using Geom = RowGeom<TPR, RB, NT>;
  constexpr int G = Geom::G;
  constexpr int WPR = Geom::WPR;
  constexpr int RPW = Geom::RPW;
  constexpr int RW = TPR < 64 ? TPR : 64;
  double* red = reinterpret_cast<double*>(dn_lds);

  const Geom geo;
  const int chunk = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = geo.lane;
  const int nvec = p.nvec;
  const bool lane_ok = TPR >= 64 || lane < nvec;
  const uint32_t row_bf16 = 2u * (uint32_t)p.hidden;
  // The chunk's rows as a strided matrix: logical row j is row chunk + j*C of the inputs.
  const int64_t C = p.chunks;
  const int64_t re = (p.rows - chunk + C - 1) / C;     // rows in this chunk
  const int64_t rb = 0;
  const uint16_t* g_c = p.g + chunk * p.sg;
  const uint16_t* x_c = p.x + chunk * p.sx;
  const uint16_t* gr_c = p.gres ? p.gres + chunk * p.sgr : nullptr;
  uint16_t* dx_c = p.dx + chunk * p.sdx;
  const float* rstd_c = p.rstd + chunk;
  const int64_t sg_c = C * p.sg, sx_c = C * p.sx, sgr_c = C * p.sgr, sdx_c = C * p.sdx;
  const double inv_hidden = 1.0 / (double)p.hidden;

  // This thread's columns are fixed for the whole chunk: weights and FP64 column sums
  // stay in registers.
  float we[VB][8];
  double acc[VB][8];
#pragma unroll
  for (int v = 0; v < VB; ++v) {
    const int idx = v * TPR + lane;
    bwd_weff8(p, idx < nvec ? idx : nvec - 1, we[v]);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[v][k] = 0.0;
  }

  // Issue every load of the step starting at row `base` (rows past the chunk read zeros).
  auto load = [&](BwdStep<VB, RB>& st, int64_t base) {
    const int64_t first = geo.first(base);
    rsrc_t rg[RB], rx[RB], rr_[RB];
    uint32_t og[RB], ox[RB], or_[RB];
    tensor_span<TPR, RB, RPW>(g_c, sg_c, 2, 16, row_bf16, first, re, lane, geo.j, lane_ok, rg,
                              og);
    tensor_span<TPR, RB, RPW>(x_c, sx_c, 2, 16, row_bf16, first, re, lane, geo.j, lane_ok, rx,
                              ox);
    if constexpr (GRES)
      tensor_span<TPR, RB, RPW>(gr_c, sgr_c, 2, 16, row_bf16, first, re, lane, geo.j,
                                lane_ok, rr_, or_);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      st.row[rr] = geo.row(first, rr);
      st.rok[rr] = st.row[rr] < re;
      st.rs[rr] = st.rok[rr] ? rstd_c[st.row[rr] * C] : 0.0f;
#pragma unroll
      for (int v = 0; v < VB; ++v) {
        const uint32_t dv = (uint32_t)(v * TPR * 16);
        st.g[rr][v] = bload16(rg[rr], og[rr] + dv);
        st.x[rr][v] = bload16(rx[rr], ox[rr] + dv);
        if constexpr (GRES) st.r[rr][v] = bload16(rr_[rr], or_[rr] + dv);
      }
    }
  };

  int parity = 0;
  // Row dot products, dx, and the FP64 column sums of one loaded step.
  auto process = [&](BwdStep<VB, RB>& st, int64_t base) {
    const int64_t first = geo.first(base);
    double dot[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      float d = 0.0f;
#pragma unroll
      for (int v = 0; v < VB; ++v) {
        float fg[8], fx[8];
        unpack8(st.g[rr][v], fg);
        unpack8(st.x[rr][v], fx);
#pragma unroll
        for (int k = 0; k < 8; ++k) d = fmaf(fg[k] * we[v][k], fx[k], d);
        keep_packed(st.g[rr][v]);
        keep_packed(st.x[rr][v]);
      }
      dot[rr] = group_sum<RW>((double)d);
    }
    if constexpr (WPR > 1) {
      const int wave_in_row = lane >> 6;
      double* slot = red + (size_t)parity * G * WPR * RB + (size_t)geo.grp * WPR * RB;
      if ((lane & 63) == 0) {
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) slot[wave_in_row * RB + rr] = dot[rr];
      }
      __syncthreads();
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        double s = 0.0;
#pragma unroll
        for (int w8 = 0; w8 < WPR; ++w8) s += slot[w8 * RB + rr];
        dot[rr] = s;
      }
      parity ^= 1;
    }
    rsrc_t rdx[RB];
    uint32_t odx[RB];
    tensor_span<TPR, RB, RPW>(dx_c, sdx_c, 2, 16, row_bf16, first, re, lane, geo.j, lane_ok,
                              rdx, odx);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      // Rows past the chunk carry r = 0 and add nothing; their dx stores are dropped.
      // dx = r * FMA(-x, r^2 * c_t, g * w_eff) [+ g_res]: the coupled coefficient carries
      // r^2, not r^3, so no factor leaves FP32's range when the row's scale is far from 1
      // (r^3 * c_t underflows FP32 for rows of RMS ~1e17 with gradients ~1e-13, and
      // overflows for rows of RMS ~1e-17 with gradients ~1e12, where dx itself is an
      // ordinary FP32 number).
      const double r64 = (double)st.rs[rr];
      const float coef = (float)(r64 * r64 * (dot[rr] * inv_hidden));
#pragma unroll
      for (int v = 0; v < VB; ++v) {
        float fg[8], fx[8], d[8];
        unpack8(st.g[rr][v], fg);
        unpack8(st.x[rr][v], fx);
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = fmaf(-fx[k], coef, fg[k] * we[v][k]);
        if constexpr (GRES) {
          float fr[8];
          unpack8(st.r[rr][v], fr);
#pragma unroll
          for (int k = 0; k < 8; ++k) d[k] = fmaf(d[k], st.rs[rr], fr[k]);
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) d[k] *= st.rs[rr];
        }
        bstore16(rdx[rr], odx[rr] + (uint32_t)(v * TPR * 16), pack8(d));
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[v][k] = fma((double)(fg[k] * fx[k]), r64, acc[v][k]);
      }
    }
  };

  if constexpr (kDB) {
    // Two steps in flight: the next step's loads are issued before the current step's
    // reduction and barrier, so the memory pipe stays busy through them.
    BwdStep<VB, RB> s0, s1;
    int64_t base = rb;
    if (base < re) load(s0, base);
    while (base < re) {
      int64_t nb = base + Geom::PER_ITER;
      if (nb < re) load(s1, nb);
      process(s0, base);
      base = nb;
      if (base >= re) break;
      nb = base + Geom::PER_ITER;
      if (nb < re) load(s0, nb);
      process(s1, base);
      base = nb;
    }
  } else {
    BwdStep<VB, RB> s0;
    for (int64_t base = rb; base < re; base += Geom::PER_ITER) {
      load(s0, base);
      process(s0, base);
    }
  }

  // The chunk's column sums: add the row groups' sums in group order, write one row.
  double* out = p.part + (int64_t)chunk * p.hidden;
  const rsrc_t orsrc = make_rsrc(out, (uint32_t)p.hidden * 8u);
  if constexpr (G == 1) {
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const int idx = v * TPR + lane;
      if (idx < nvec) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          bstore16_p<kChunkStorePolicy>(
              orsrc, (uint32_t)(idx * 64 + 16 * k),
              __builtin_bit_cast(v4u, make_double2(acc[v][2 * k], acc[v][2 * k + 1])));
      }
    }
  } else {
    __syncthreads();                       // the dot-product slots are reused below
    constexpr int GV = TPR * VB;           // column vectors held by one row group
    double* comb = red;                    // [G][GV][kCombPitch]
#pragma unroll
    for (int v = 0; v < VB; ++v)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        comb[((size_t)geo.grp * GV + v * TPR + lane) * kCombPitch + k] = acc[v][k];
    __syncthreads();
    for (int col = tid; col < p.hidden; col += NT) {
      double s = 0.0;
      for (int gg = 0; gg < G; ++gg) s += comb[((size_t)gg * GV + (col >> 3)) * kCombPitch + (col & 7)];
      bstore8_p<kChunkStorePolicy>(orsrc, (uint32_t)col * 8u, __builtin_bit_cast(v2u, s));
    }
  }

}

// (threads per row, vectors per thread, rows per group per step, threads per block).
// The host takes the first tier, in this order, whose TPR*VB covers hidden/8; the tiers
// after the tenth are alternatives for tuning builds.  Rows of 65-1024 vectors (H 520 to
// 8192) take several row groups per block (four groups of 64 lanes in a 256-thread block,
// 2 vectors per lane up to H = 1024 and 4 up to 2048; four of 128 lanes up to 4096 and two
// of 256 lanes up to 8192, 4 vectors each, in a 512-thread block): the chunk's rows
// alternate between the groups, each group keeps its own FP64 column sums, and they are
// added in group order at the end (through 32-128 KiB of LDS).  Measured against one row
// group of 1-2 vectors per
// lane with several rows per step: at H = 8192 +3.4 % at 16384 rows (+3 % with a
// residual gradient), +3.7 % at 4096, +7 % at 2048; at H = 4096 +7 %, +7 % and +2 %
// (+4 % with a residual gradient); at H = 2048 +12 %, +6 % and +3 % (+8 %).  At H = 1024
// four groups of 64 lanes with 2 vectors and 2 rows per step: +15 %, +4 % and +3 % (+13 %,
// +5.5 %, -1 % with a residual gradient; 32 lanes with 4 vectors lost 3-4 % at 2048-4096
// rows).  Wider rows span the whole block.
#define DN_BWD_TIERS(X)                                                         \
  X(0, 8, 1, 4, 256)     X(1, 16, 1, 4, 256)    X(2, 32, 1, 4, 256)            \
  X(3, 64, 1, 4, 256)    X(4, 64, 2, 2, 256)    X(5, 64, 4, 1, 256)            \
  X(6, 128, 4, 1, 512)   X(7, 256, 4, 1, 512)   X(8, 512, 4, 1, 512)           \
  X(9, 1024, 4, 1, 1024) X(10, 1024, 1, 4, 1024) X(11, 512, 2, 4, 512)         \
  X(12, 1024, 1, 2, 1024) X(13, 512, 1, 2, 512) X(14, 512, 2, 2, 512)           \
  X(15, 512, 1, 4, 512)  X(16, 256, 1, 4, 256)  X(17, 128, 1, 4, 256)

constexpr int kBwdTierCount = 18;

}  // namespace dn
