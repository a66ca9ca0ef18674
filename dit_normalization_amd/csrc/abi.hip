// C ABI of the RMSNorm and LayerNorm families (include/dnorm.h): host-side argument checks, row-tier
// selection by hidden size, persistent-grid sizing, and the kernel launches.
//
// Every check runs before the first HIP call, so a rejected call touches no device state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "dn_launch.h"
#include "dnorm.h"

using namespace dn;

namespace {

constexpr int kMaxHidden = 32768;
// Row strides are bounded so that the rows one wave touches in a step (at most 32) span
// less than 2^30 bytes: buffer descriptors carry 32-bit record counts.
constexpr int64_t kMaxStride = (int64_t)1 << 24;
// Per-column parameters are staged in LDS up to this many 16-byte column vectors (32 KiB
// of FP32 per block for the RMSNorm weight, 64 KiB for LayerNorm gamma and beta); wider
// rows read them from global memory (L2-resident) instead.
constexpr int kMaxLdsWeightVectors = 1024;

// Persistent forward grids hold at most DN_BLOCKS_PER_CU blocks per compute unit: on
// MI355X fewer streams in flight keep HBM more efficient (measured 2 blocks of 256 threads
// per CU ahead of full occupancy) when a row reads two or more tensors.  Kernels that
// stream a single input tensor keep too few bytes in flight that way and take up to
// DN_BLOCKS_PER_CU_SINGLE (measured at [8192, 4096]: static-FP8 RMSNorm 3.70 -> 4.39 TB/s,
// LayerNorm 4.23 -> 4.62 TB/s with 4).  Tuning builds can override both (0 = as many as
// are resident) and the backward row tier (-1 = by hidden size).
#ifndef DN_BLOCKS_PER_CU
#define DN_BLOCKS_PER_CU 2
#endif
#ifndef DN_BLOCKS_PER_CU_SINGLE
#define DN_BLOCKS_PER_CU_SINGLE 4
#endif
// The SiLU and sigmoid-gate epilogues are latency-bound (the vector ALUs about half busy,
// HBM about half used), so they take all eight blocks a CU holds: more waves to cover each
// other's memory waits and exp/rcp chains (measured: SiLU + FP8 +4 to +13 % and SiLU +2 to
// +4 % at the video-VAE shapes against 4 blocks; the per-head sigmoid gate +2 to +3.5 %
// against 2).
#ifndef DN_BLOCKS_PER_CU_VALU
#define DN_BLOCKS_PER_CU_VALU 8
#endif
#ifndef DN_BWD_TIER
#define DN_BWD_TIER -1
#endif

thread_local std::string g_error;
std::atomic<int> g_force_tpr{0};

dn_status fail(dn_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

dn_status check_shape(int64_t rows, int64_t hidden, int64_t multiple, const char* what) {
  if (rows < 0) return fail(DN_ERR_SHAPE, "rows must be >= 0 (got %lld)", (long long)rows);
  if (hidden <= 0 || hidden > kMaxHidden)
    return fail(DN_ERR_SHAPE, "%s must be in [1, %d] (got %lld)", what, kMaxHidden,
                (long long)hidden);
  if (hidden % multiple != 0)
    return fail(DN_ERR_UNSUPPORTED, "%s must be a multiple of %lld (got %lld)", what,
                (long long)multiple, (long long)hidden);
  return DN_OK;
}

// A [rows, hidden] matrix of BF16 (elem = 2) or FP8 (elem = 1) with a row stride in
// elements: 16-byte vectors of the row must stay aligned.
dn_status check_matrix(const void* p, int64_t stride, int64_t hidden, int elem,
                       const char* name) {
  if (!p) return fail(DN_ERR_NULL, "%s must not be NULL", name);
  if (stride < hidden)
    return fail(DN_ERR_SHAPE, "%s row stride %lld is smaller than the row width %lld", name,
                (long long)stride, (long long)hidden);
  const size_t base_align = elem == 2 ? 16 : 8;
  if (!aligned(p, base_align))
    return fail(DN_ERR_ALIGN, "%s must be %zu-byte aligned", name, base_align);
  if (stride % 8 != 0)
    return fail(DN_ERR_ALIGN, "%s row stride %lld must be a multiple of 8 elements", name,
                (long long)stride);
  if (stride > kMaxStride)
    return fail(DN_ERR_SHAPE, "%s row stride %lld exceeds %lld elements", name,
                (long long)stride, (long long)kMaxStride);
  return DN_OK;
}

dn_status check_weight(const void* w, int w_dtype) {
  if (w_dtype != DN_WEIGHT_BF16 && w_dtype != DN_WEIGHT_F32)
    return fail(DN_ERR_DTYPE, "w_dtype must be DN_WEIGHT_BF16 (0) or DN_WEIGHT_F32 (1), got %d",
                w_dtype);
  if (!w) return fail(DN_ERR_NULL, "w must not be NULL");
  if (!aligned(w, 16)) return fail(DN_ERR_ALIGN, "w must be 16-byte aligned");
  return DN_OK;
}

dn_status check_f32(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(DN_ERR_NULL, "%s must not be NULL", name) : DN_OK;
  if (!aligned(p, 4)) return fail(DN_ERR_ALIGN, "%s must be 4-byte aligned", name);
  return DN_OK;
}

#define DN_CHECK(expr)              \
  do {                              \
    const dn_status s_ = (expr);    \
    if (s_ != DN_OK) return s_;     \
  } while (0)

// ------------------------------------------------------------------ device properties

struct DeviceCache {
  std::mutex mu;
  std::map<int, int> cus;
  std::map<std::tuple<int, const void*, size_t, int>, int> occ;
};

DeviceCache& cache() {
  static DeviceCache c;
  return c;
}

dn_status resident_blocks(const void* kernel, int nt, size_t lds, int cap, int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DN_ERR_HIP, "hipGetDevice failed");
  DeviceCache& c = cache();
  std::lock_guard<std::mutex> lock(c.mu);
  auto it = c.cus.find(dev);
  if (it == c.cus.end()) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return fail(DN_ERR_HIP, "cannot read the compute-unit count of device %d", dev);
    it = c.cus.emplace(dev, n).first;
  }
  const auto key = std::make_tuple(dev, kernel, lds, cap);
  auto ot = c.occ.find(key);
  if (ot == c.occ.end()) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, nt, lds) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    if (cap > 0 && per_cu > cap) per_cu = cap;
#ifdef DN_WAVES_PER_CU
    {
      const int cap = DN_WAVES_PER_CU * 64 / nt;
      per_cu = std::min(per_cu, cap > 0 ? cap : 1);
    }
#endif
    ot = c.occ.emplace(key, per_cu).first;
  }
  *out = it->second * ot->second;
  return DN_OK;
}

// Grid of a persistent row kernel that needs `needed` block-steps.  Normally at most `cap`
// blocks per CU (fewer bytes in flight stream better); but when that leaves each block
// fewer than `tail_steps` steps, the ramp and the last, partly filled round of steps weigh
// on the launch, so every block-step is put in flight at once as far as occupancy allows
// (up to kTailBlocksPerCu blocks per CU).  Measured: gated Ada + FP8 at [2520,3072] 4.96
// -> 5.27 TB/s, fused add at [2520,4096] 4.63 -> 5.56 TB/s (fewer than three steps); with
// the threshold raised from three to five steps, fused add (+ static FP8) at [4096,4096]
// +12-13 %, block quant at [2048,7168] +8 %, gated Ada + FP8 at [4096,3072] +4 %, the
// training forward of the [2048,8192] shard +3 %, the DiT modes at [4096,3072] -0.7 %.
// At seven steps the DiT modes lost 3 % (at [6144,3072]), so launches of five or more
// steps per block keep the cap.  The fused add with a static FP8 output (a lighter write
// share than the BF16 forms) gains from full occupancy up to eight steps per block: fused
// add + FP8 [8192,4096] +3.8 %, [6144,4096] +6.8 %, per head [8192,32,128] +5.9 %,
// unchanged at twelve steps; the single-input rmsnorm_quant lost 1.8 % at eight steps.
constexpr int kTailBlocksPerCu = 8;
constexpr int kTailSteps = 5;
constexpr int kTailStepsAddFp8 = 9;

dn_status persistent_grid(const void* kernel, int nt, size_t lds, int cap, int64_t needed,
                          int* grid, int tail_steps = kTailSteps) {
  int capacity = 0;
  DN_CHECK(resident_blocks(kernel, nt, lds, cap, &capacity));
  if (needed < tail_steps * (int64_t)capacity) {
    int full = 0;
    DN_CHECK(resident_blocks(kernel, nt, lds, kTailBlocksPerCu, &full));
    if (full > capacity) capacity = full;
  }
  const int64_t g = needed < capacity ? needed : capacity;
  *grid = g > 0 ? (int)g : 1;
  return DN_OK;
}

// ------------------------------------------------------------------ forward dispatch

int pick_fwd_tier(int nvec, int limit, int forced) {
  const int count = forced ? kFwdTierCount : kFwdAutoTiers;
  for (int t = 0; t < count; ++t) {
    const TierShape s = fwd_tier_shape(t);
    if (s.vmax > limit || s.tpr * s.vmax < nvec) continue;
    if (forced && s.tpr != forced) continue;
    return t;
  }
  return forced ? pick_fwd_tier(nvec, limit, 0) : -1;
}

template <int IN, int EPI>
dn_status launch_fwd(FwdParams p, hipStream_t stream) {
  p.nvec = p.hidden / 8;
  const int tier = pick_fwd_tier(p.nvec, fwd_vmax_limit(IN, EPI), g_force_tpr.load());
  if (tier < 0) return fail(DN_ERR_SHAPE, "hidden %d is too wide", p.hidden);
  const TierShape s = fwd_tier_shape(tier);
  const int g = s.nt / s.tpr;
  const int wpr = s.tpr > 64 ? s.tpr / 64 : 1;
  constexpr int planes = fwd_weight_planes(EPI);
  p.w_in_lds = planes > 0 && p.nvec <= kMaxLdsWeightVectors;
  const size_t lds = fwd_lds_bytes(p.nvec, p.w_in_lds ? planes : 0, g, wpr, s.r, fwd_stats(EPI));

  const void* kernel = nullptr;
  if (fwd_launch<IN, EPI>(p, tier, 0, 0, nullptr, &kernel) != hipSuccess || !kernel)
    return fail(DN_ERR_HIP, "no kernel instance for tier %d", tier);
  constexpr bool single_stream = IN == IN_PLAIN && EPI != EPI_ADA_BF16 &&
                                 EPI != EPI_ADA_FP8 && EPI != EPI_LN_MOD_BF16 &&
                                 EPI != EPI_SIGMOID_GATE;
  constexpr bool valu_heavy = epi_is_silu(EPI) || EPI == EPI_SIGMOID_GATE;
  const int64_t per_iter = (int64_t)g * s.r;
  const int64_t needed = (p.rows + per_iter - 1) / per_iter;
  const int cap = valu_heavy      ? DN_BLOCKS_PER_CU_VALU
                  : single_stream ? DN_BLOCKS_PER_CU_SINGLE
                                  : DN_BLOCKS_PER_CU;
  int grid = 0;
  constexpr int tail_steps = IN == IN_ADD && EPI == EPI_FP8 ? kTailStepsAddFp8 : kTailSteps;
  DN_CHECK(persistent_grid(kernel, s.nt, lds, cap, needed, &grid, tail_steps));
  const hipError_t e = fwd_launch<IN, EPI>(p, tier, grid, lds, stream, nullptr);
  if (e != hipSuccess) return fail(DN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return DN_OK;
}

FwdParams base_params(int64_t rows, int64_t hidden, float eps) {
  FwdParams p{};
  p.rows = rows;
  p.hidden = (int)hidden;
  p.eps = eps;
  return p;
}

// ------------------------------------------------------------------ backward dispatch

int pick_bwd_tier(int nvec) {
  if (DN_BWD_TIER >= 0 && DN_BWD_TIER < kBwdTierCount) {
    const TierShape s = bwd_tier_shape(DN_BWD_TIER);
    if (s.tpr * s.vmax >= nvec) return DN_BWD_TIER;
  }
  for (int t = 0; t < kBwdTierCount; ++t) {
    const TierShape s = bwd_tier_shape(t);
    if (s.tpr * s.vmax >= nvec) return t;
  }
  return -1;
}

// Workspace: kMaxChunks rows of FP64 column sums.
size_t workspace_bytes(int64_t hidden) {
  if (hidden <= 0 || hidden > kMaxHidden) return 0;
  return (size_t)kMaxChunks * (size_t)hidden * sizeof(double);
}

dn_status check_workspace(const void* ws, size_t bytes, int64_t hidden) {
  if (!ws) return fail(DN_ERR_NULL, "workspace must not be NULL");
  if (!aligned(ws, 256)) return fail(DN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = workspace_bytes(hidden);
  if (bytes < need)
    return fail(DN_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed for hidden %lld", bytes,
                need, (long long)hidden);
  return DN_OK;
}

int chunk_count(int64_t rows) { return (int)(rows < kMaxChunks ? rows : kMaxChunks); }

// LayerNorm gamma and beta: FP32 [hidden], 16-byte aligned.
dn_status check_affine(const float* gamma, const float* beta) {
  if (!gamma) return fail(DN_ERR_NULL, "gamma must not be NULL");
  if (!beta) return fail(DN_ERR_NULL, "beta must not be NULL");
  if (!aligned(gamma, 16)) return fail(DN_ERR_ALIGN, "gamma must be 16-byte aligned");
  if (!aligned(beta, 16)) return fail(DN_ERR_ALIGN, "beta must be 16-byte aligned");
  return DN_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

const char* dn_last_error(void) { return g_error.c_str(); }

int dn_max_hidden(void) { return kMaxHidden; }

const char* dn_version(void) { return "dnorm 0.1 (gfx950)"; }

dn_status dn_force_threads_per_row(int threads) {
  switch (threads) {
    case 0: case 8: case 16: case 32: case 64: case 128: case 256: case 320: case 448:
    case 512: case 1024:
      g_force_tpr.store(threads);
      return DN_OK;
    default:
      return fail(DN_ERR_SHAPE,
                  "threads per row must be 0, a power of two in [8, 1024], 320 or 448");
  }
}

dn_status dn_rmsnorm(void* y, int64_t y_stride, float* rstd, const void* x, int64_t x_stride,
                     const void* w, int w_dtype, float w_bias, int64_t rows, int64_t hidden,
                     float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(y, y_stride, hidden, 2, "y"));
  DN_CHECK(check_weight(w, w_dtype));
  DN_CHECK(check_f32(rstd, "rstd", false));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.y = static_cast<uint16_t*>(y); p.sy = y_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  p.rstd = rstd;
  return launch_fwd<IN_PLAIN, EPI_BF16>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_rmsnorm_quant(uint8_t* out, int64_t out_stride, const void* x, int64_t x_stride,
                           const void* w, int w_dtype, float w_bias, const float* scale,
                           int64_t rows, int64_t hidden, float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(out, out_stride, hidden, 1, "out"));
  DN_CHECK(check_weight(w, w_dtype));
  DN_CHECK(check_f32(scale, "scale", true));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.q = out; p.sq = out_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  p.scale = scale;
  return launch_fwd<IN_PLAIN, EPI_FP8>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_fused_add_rmsnorm(void* x, int64_t x_stride, void* residual,
                               int64_t residual_stride, const void* w, int w_dtype,
                               float w_bias, float* rstd, int64_t rows, int64_t hidden,
                               float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
  DN_CHECK(check_weight(w, w_dtype));
  DN_CHECK(check_f32(rstd, "rstd", false));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.h = static_cast<uint16_t*>(residual); p.sh = residual_stride;
  p.y = static_cast<uint16_t*>(x); p.sy = x_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  p.rstd = rstd;
  return launch_fwd<IN_ADD, EPI_BF16>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_fused_add_rmsnorm_quant(uint8_t* out, int64_t out_stride, const void* x,
                                     int64_t x_stride, void* residual, int64_t residual_stride,
                                     const void* w, int w_dtype, float w_bias,
                                     const float* scale, int64_t rows, int64_t hidden,
                                     float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
  DN_CHECK(check_matrix(out, out_stride, hidden, 1, "out"));
  DN_CHECK(check_weight(w, w_dtype));
  DN_CHECK(check_f32(scale, "scale", true));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.h = static_cast<uint16_t*>(residual); p.sh = residual_stride;
  p.q = out; p.sq = out_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  p.scale = scale;
  return launch_fwd<IN_ADD, EPI_FP8>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_fused_add_rmsnorm_fp8_block_quant(uint8_t* out, int64_t out_stride,
                                               float* block_scale, int64_t scale_ld,
                                               void* normed_out, int64_t normed_stride,
                                               const void* x, int64_t x_stride, void* residual,
                                               int64_t residual_stride, const void* w,
                                               int w_dtype, float w_bias, int64_t rows,
                                               int64_t hidden, float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 128, "hidden (1x128 blocks)"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
  DN_CHECK(check_matrix(out, out_stride, hidden, 1, "out"));
  if (normed_out) DN_CHECK(check_matrix(normed_out, normed_stride, hidden, 2, "normed_out"));
  DN_CHECK(check_weight(w, w_dtype));
  DN_CHECK(check_f32(block_scale, "block_scale", true));
  if (scale_ld < rows)
    return fail(DN_ERR_SHAPE, "scale_ld %lld is smaller than rows %lld", (long long)scale_ld,
                (long long)rows);
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.h = static_cast<uint16_t*>(residual); p.sh = residual_stride;
  p.y = static_cast<uint16_t*>(normed_out); p.sy = normed_stride;
  p.q = out; p.sq = out_stride;
  p.bscale = block_scale; p.bld = scale_ld;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  return launch_fwd<IN_ADD, EPI_FP8_BLOCK>(p, static_cast<hipStream_t>(stream));
}

static dn_status check_style(const void* style, int64_t style_stride, int64_t style_rows,
                             int64_t rows, int64_t dim) {
  if (!style) return fail(DN_ERR_NULL, "style must not be NULL");
  if (style_rows != 1 && style_rows != rows)
    return fail(DN_ERR_SHAPE, "style_rows must be 1 or rows (%lld), got %lld", (long long)rows,
                (long long)style_rows);
  return check_matrix(style, style_stride, 3 * dim, 2, "style");
}

dn_status dn_ada_rms_norm(void* out, int64_t out_stride, void* gate_out,
                          int64_t gate_out_stride, const void* x, int64_t x_stride,
                          const void* w, const void* style, int64_t style_stride,
                          int64_t style_rows, int64_t rows, int64_t dim, float eps,
                          dn_stream_t stream) {
  DN_CHECK(check_shape(rows, dim, 8, "dim"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, dim, 2, "x"));
  DN_CHECK(check_matrix(out, out_stride, dim, 2, "out"));
  if (gate_out) DN_CHECK(check_matrix(gate_out, gate_out_stride, dim, 2, "gate_out"));
  DN_CHECK(check_weight(w, DN_WEIGHT_BF16));
  DN_CHECK(check_style(style, style_stride, style_rows, rows, dim));
  FwdParams p = base_params(rows, dim, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.y = static_cast<uint16_t*>(out); p.sy = out_stride;
  p.gate_out = static_cast<uint16_t*>(gate_out); p.sgo = gate_out_stride;
  p.style = static_cast<const uint16_t*>(style); p.sst = style_stride;
  p.style_bcast = style_rows == 1;
  p.w = w; p.w_f32 = 0; p.w_bias = 0.0f;
  return launch_fwd<IN_PLAIN, EPI_ADA_BF16>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_gate_residual_ada_norm_fp8(void* residual, int64_t residual_stride, uint8_t* out,
                                        int64_t out_stride, void* gate_out,
                                        int64_t gate_out_stride, const void* x,
                                        int64_t x_stride, const void* gate, int64_t gate_stride,
                                        const void* w, const void* style, int64_t style_stride,
                                        int64_t style_rows, const float* scale, int64_t rows,
                                        int64_t dim, float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, dim, 8, "dim"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(residual, residual_stride, dim, 2, "residual"));
  DN_CHECK(check_matrix(x, x_stride, dim, 2, "x"));
  DN_CHECK(check_matrix(gate, gate_stride, dim, 2, "gate"));
  DN_CHECK(check_matrix(out, out_stride, dim, 1, "out"));
  if (gate_out) DN_CHECK(check_matrix(gate_out, gate_out_stride, dim, 2, "gate_out"));
  DN_CHECK(check_weight(w, DN_WEIGHT_BF16));
  DN_CHECK(check_style(style, style_stride, style_rows, rows, dim));
  DN_CHECK(check_f32(scale, "scale", true));
  FwdParams p = base_params(rows, dim, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.gate = static_cast<const uint16_t*>(gate); p.sg = gate_stride;
  p.h = static_cast<uint16_t*>(residual); p.sh = residual_stride;
  p.q = out; p.sq = out_stride;
  p.gate_out = static_cast<uint16_t*>(gate_out); p.sgo = gate_out_stride;
  p.style = static_cast<const uint16_t*>(style); p.sst = style_stride;
  p.style_bcast = style_rows == 1;
  p.w = w; p.w_f32 = 0; p.w_bias = 0.0f;
  p.scale = scale;
  return launch_fwd<IN_GATED, EPI_ADA_FP8>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_train_forward(void* y, int64_t y_stride, float* rstd, void* h_new,
                           int64_t h_new_stride, const void* x, int64_t x_stride,
                           const void* residual, int64_t residual_stride, const void* w,
                           int w_dtype, float w_bias, int64_t rows, int64_t hidden, float eps,
                           dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(y, y_stride, hidden, 2, "y"));
  DN_CHECK(check_weight(w, w_dtype));
  DN_CHECK(check_f32(rstd, "rstd", true));
  if (residual) {
    DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
    DN_CHECK(check_matrix(h_new, h_new_stride, hidden, 2, "h_new"));
  }
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.y = static_cast<uint16_t*>(y); p.sy = y_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  p.rstd = rstd;
  if (!residual) return launch_fwd<IN_PLAIN, EPI_BF16>(p, static_cast<hipStream_t>(stream));
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.h = static_cast<uint16_t*>(h_new); p.sh = h_new_stride;
  return launch_fwd<IN_ADD, EPI_BF16>(p, static_cast<hipStream_t>(stream));
}

size_t dn_train_backward_workspace_bytes(int64_t hidden) { return workspace_bytes(hidden); }

namespace {

dn_status check_dw(const void* dw, int dw_dtype) {
  if (dw_dtype != DN_WEIGHT_BF16 && dw_dtype != DN_WEIGHT_F32)
    return fail(DN_ERR_DTYPE, "dw_dtype must be DN_WEIGHT_BF16 (0) or DN_WEIGHT_F32 (1), got %d",
                dw_dtype);
  if (!dw) return fail(DN_ERR_NULL, "dw must not be NULL");
  if (!aligned(dw, dw_dtype == DN_WEIGHT_F32 ? 4 : 2))
    return fail(DN_ERR_ALIGN, "dw must be %d-byte aligned", dw_dtype == DN_WEIGHT_F32 ? 4 : 2);
  return DN_OK;
}

// Checks of the backward's row arguments and the BwdParams of a producer launch over
// `part` (chunk rows) and `ctr` (counters, one-launch form).  *tier_out receives the row
// tier.  rows == 0 is handled by the caller.
dn_status bwd_prepare(BwdParams* out, int* tier_out, void* dx, int64_t dx_stride, const void* g,
                      int64_t g_stride, const void* x, int64_t x_stride, const void* w,
                      int w_dtype, float w_bias, const float* rstd, const void* g_residual,
                      int64_t g_residual_stride, int64_t rows, int64_t hidden) {
  DN_CHECK(check_matrix(dx, dx_stride, hidden, 2, "dx"));
  DN_CHECK(check_matrix(g, g_stride, hidden, 2, "g"));
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  if (g_residual) DN_CHECK(check_matrix(g_residual, g_residual_stride, hidden, 2, "g_residual"));
  DN_CHECK(check_weight(w, w_dtype));
  DN_CHECK(check_f32(rstd, "rstd", true));
  BwdParams p{};
  p.dx = static_cast<uint16_t*>(dx); p.sdx = dx_stride;
  p.g = static_cast<const uint16_t*>(g); p.sg = g_stride;
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.gres = static_cast<const uint16_t*>(g_residual); p.sgr = g_residual_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  p.rstd = rstd;
  p.rows = rows;
  p.hidden = (int)hidden;
  p.nvec = (int)(hidden / 8);
  p.chunks = chunk_count(rows);
  const int tier = pick_bwd_tier(p.nvec);
  if (tier < 0) return fail(DN_ERR_SHAPE, "hidden %lld is too wide", (long long)hidden);
  // A chunk's rows are every C-th row: rows that share a wave span (narrow rows) sit
  // C row strides apart, and the span's byte range must stay below 2^30.
  if (bwd_tier_shape(tier).tpr < 64) {
    const int64_t widest = std::max(std::max(dx_stride, g_stride),
                                    std::max(x_stride, g_residual ? g_residual_stride : 0));
    if ((int64_t)32 * p.chunks * widest * 2 >= ((int64_t)1 << 30))
      return fail(DN_ERR_SHAPE, "row strides up to %lld elements are supported at hidden %lld",
                  (long long)(((int64_t)1 << 30) / (64 * p.chunks) - 1), (long long)hidden);
  }
  *out = p;
  *tier_out = tier;
  return DN_OK;
}

// Launch the producers of `p` (dx and the chunk rows in p.part); with `dw`, also the
// reduction of the chunk rows into dw on the same stream.
dn_status bwd_launch(const BwdParams& p, int tier, void* dw, int dw_dtype,
                     hipStream_t stream) {
  const TierShape s = bwd_tier_shape(tier);
  const int gcount = s.nt / s.tpr;
  const int wpr = s.tpr > 64 ? s.tpr / 64 : 1;
  const size_t lds = bwd_lds_bytes(gcount, wpr, s.r, s.nt, s.vmax);
  hipError_t e = bwd_partials_launch(p, tier, lds, stream, nullptr);
  if (e == hipSuccess && dw)
    e = bwd_reduce_launch(dw, dw_dtype == DN_WEIGHT_BF16, p.part, p.hidden, p.chunks, stream);
  if (e != hipSuccess) return fail(DN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return DN_OK;
}

}  // namespace

dn_status dn_train_backward_partials(void* dx, int64_t dx_stride, const void* g,
                                     int64_t g_stride, const void* x, int64_t x_stride,
                                     const void* w, int w_dtype, float w_bias,
                                     const float* rstd, const void* g_residual,
                                     int64_t g_residual_stride, void* workspace,
                                     size_t workspace_bytes_, int64_t rows, int64_t hidden,
                                     dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  BwdParams p;
  int tier = 0;
  DN_CHECK(bwd_prepare(&p, &tier, dx, dx_stride, g, g_stride, x, x_stride, w, w_dtype, w_bias,
                       rstd, g_residual, g_residual_stride, rows, hidden));
  DN_CHECK(check_workspace(workspace, workspace_bytes_, hidden));
  p.part = static_cast<double*>(workspace);
  return bwd_launch(p, tier, nullptr, 0, static_cast<hipStream_t>(stream));
}

dn_status dn_train_backward_reduce(void* dw, int dw_dtype, const void* workspace,
                                   size_t workspace_bytes_, int64_t rows, int64_t hidden,
                                   dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_dw(dw, dw_dtype));
  DN_CHECK(check_workspace(workspace, workspace_bytes_, hidden));
  const hipError_t e = bwd_reduce_launch(dw, dw_dtype == DN_WEIGHT_BF16,
                                         static_cast<const double*>(workspace), (int)hidden,
                                         chunk_count(rows), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return DN_OK;
}

dn_status dn_train_backward(void* dx, int64_t dx_stride, void* dw, int dw_dtype, const void* g,
                            int64_t g_stride, const void* x, int64_t x_stride, const void* w,
                            int w_dtype, float w_bias, const float* rstd,
                            const void* g_residual, int64_t g_residual_stride,
                            void* workspace, size_t workspace_bytes_, int64_t rows,
                            int64_t hidden, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_dw(dw, dw_dtype));
  BwdParams p;
  int tier = 0;
  DN_CHECK(bwd_prepare(&p, &tier, dx, dx_stride, g, g_stride, x, x_stride, w, w_dtype, w_bias,
                       rstd, g_residual, g_residual_stride, rows, hidden));
  DN_CHECK(check_workspace(workspace, workspace_bytes_, hidden));
  p.part = static_cast<double*>(workspace);
  return bwd_launch(p, tier, dw, dw_dtype, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ allocation-free backward

namespace {

// Scratch of dn_train_backward_noalloc: the FP64 chunk rows for hidden up to
// kNoAllocMaxHidden.  Every GPU the library runs on holds its own copy (16 MiB) until the
// process ends.
constexpr int64_t kNoAllocMaxHidden = 8192;
constexpr size_t kScratchBytes = (size_t)kMaxChunks * kNoAllocMaxHidden * sizeof(double);

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The device address of `scratch` on the current device, looked up once per device (the
// host-side name is only a stand-in for it).  Nothing in it needs clearing: every call
// rewrites the chunk rows it reads.
dn_status scratch_address(unsigned char** out) {
  static std::mutex mu;
  static std::map<int, unsigned char*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DN_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it != ptrs.end()) {
    *out = it->second;
    return DN_OK;
  }
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(DN_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(e));
  *out = static_cast<unsigned char*>(ptr);
  ptrs.emplace(dev, *out);
  return DN_OK;
}

}  // namespace

dn_status dn_train_backward_noalloc(void* dx, int64_t dx_stride, void* dw, int dw_dtype,
                                    const void* g, int64_t g_stride, const void* x,
                                    int64_t x_stride, const void* w, int w_dtype, float w_bias,
                                    const float* rstd, const void* g_residual,
                                    int64_t g_residual_stride, int64_t rows, int64_t hidden,
                                    dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (hidden > kNoAllocMaxHidden)
    return fail(DN_ERR_UNSUPPORTED,
                "hidden %lld exceeds the allocation-free scratch (hidden <= %lld); use "
                "dn_train_backward with a workspace", (long long)hidden,
                (long long)kNoAllocMaxHidden);
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_dw(dw, dw_dtype));
  BwdParams p;
  int tier = 0;
  DN_CHECK(bwd_prepare(&p, &tier, dx, dx_stride, g, g_stride, x, x_stride, w, w_dtype, w_bias,
                       rstd, g_residual, g_residual_stride, rows, hidden));
  unsigned char* base = nullptr;
  DN_CHECK(scratch_address(&base));
  p.part = reinterpret_cast<double*>(base);
  return bwd_launch(p, tier, dw, dw_dtype, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ LayerNorm family

dn_status dn_layernorm(void* y, int64_t y_stride, const void* x, int64_t x_stride,
                       const float* gamma, const float* beta, int64_t rows, int64_t hidden,
                       float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(y, y_stride, hidden, 2, "y"));
  DN_CHECK(check_affine(gamma, beta));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.y = static_cast<uint16_t*>(y); p.sy = y_stride;
  p.w = gamma; p.w_f32 = 1; p.beta = beta;
  return launch_fwd<IN_PLAIN, EPI_LN_BF16>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_layernorm_quant(uint8_t* out, int64_t out_stride, const void* x, int64_t x_stride,
                             const float* gamma, const float* beta, const float* scale,
                             int64_t rows, int64_t hidden, float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(out, out_stride, hidden, 1, "out"));
  DN_CHECK(check_affine(gamma, beta));
  DN_CHECK(check_f32(scale, "scale", true));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.q = out; p.sq = out_stride;
  p.w = gamma; p.w_f32 = 1; p.beta = beta;
  p.scale = scale;
  return launch_fwd<IN_PLAIN, EPI_LN_FP8>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_fused_dit_gate_residual_layernorm_gamma_beta(
    void* residual_out, int64_t residual_out_stride, void* norm_out, int64_t norm_out_stride,
    const void* x, int64_t x_stride, const void* residual, int64_t residual_stride,
    const void* gate, int64_t gate_stride, float gate_bias, const float* gamma,
    const float* beta, int64_t rows, int64_t hidden, float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
  DN_CHECK(check_matrix(gate, gate_stride, hidden, 2, "gate"));
  DN_CHECK(check_matrix(norm_out, norm_out_stride, hidden, 2, "norm_out"));
  if (residual_out)
    DN_CHECK(check_matrix(residual_out, residual_out_stride, hidden, 2, "residual_out"));
  DN_CHECK(check_affine(gamma, beta));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.gate = static_cast<const uint16_t*>(gate); p.sg = gate_stride;
  p.gate_bias = gate_bias;
  p.h = static_cast<uint16_t*>(residual_out); p.sh = residual_out_stride;
  p.y = static_cast<uint16_t*>(norm_out); p.sy = norm_out_stride;
  p.w = gamma; p.w_f32 = 1; p.beta = beta;
  return launch_fwd<IN_GATED_BIAS, EPI_LN_BF16>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_fused_dit_gate_residual_layernorm_scale_shift(
    void* residual_out, int64_t residual_out_stride, void* norm_out, int64_t norm_out_stride,
    const void* x, int64_t x_stride, const void* residual, int64_t residual_stride,
    const void* gate, int64_t gate_stride, float gate_bias, const void* scale,
    int64_t scale_stride, float scale_bias, const void* shift, int64_t shift_stride,
    float shift_bias, int64_t rows, int64_t hidden, float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
  DN_CHECK(check_matrix(gate, gate_stride, hidden, 2, "gate"));
  DN_CHECK(check_matrix(scale, scale_stride, hidden, 2, "scale"));
  DN_CHECK(check_matrix(shift, shift_stride, hidden, 2, "shift"));
  DN_CHECK(check_matrix(norm_out, norm_out_stride, hidden, 2, "norm_out"));
  if (residual_out)
    DN_CHECK(check_matrix(residual_out, residual_out_stride, hidden, 2, "residual_out"));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.gate = static_cast<const uint16_t*>(gate); p.sg = gate_stride;
  p.gate_bias = gate_bias;
  p.msc = static_cast<const uint16_t*>(scale); p.smsc = scale_stride;
  p.msh = static_cast<const uint16_t*>(shift); p.smsh = shift_stride;
  p.scale_bias = scale_bias; p.shift_bias = shift_bias;
  p.h = static_cast<uint16_t*>(residual_out); p.sh = residual_out_stride;
  p.y = static_cast<uint16_t*>(norm_out); p.sy = norm_out_stride;
  return launch_fwd<IN_GATED_BIAS, EPI_LN_MOD_BF16>(p, static_cast<hipStream_t>(stream));
}

dn_status dn_fused_dit_residual_layernorm_scale_shift(
    void* residual_out, int64_t residual_out_stride, void* norm_out, int64_t norm_out_stride,
    const void* x, int64_t x_stride, const void* residual, int64_t residual_stride,
    const void* scale, int64_t scale_stride, float scale_bias, const void* shift,
    int64_t shift_stride, float shift_bias, int64_t rows, int64_t hidden, float eps,
    dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(scale, scale_stride, hidden, 2, "scale"));
  DN_CHECK(check_matrix(shift, shift_stride, hidden, 2, "shift"));
  DN_CHECK(check_matrix(norm_out, norm_out_stride, hidden, 2, "norm_out"));
  if (residual) {
    DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
    if (residual_out)
      DN_CHECK(check_matrix(residual_out, residual_out_stride, hidden, 2, "residual_out"));
  } else if (residual_out) {
    return fail(DN_ERR_UNSUPPORTED, "residual_out needs a residual (pass NULL for both)");
  }
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.msc = static_cast<const uint16_t*>(scale); p.smsc = scale_stride;
  p.msh = static_cast<const uint16_t*>(shift); p.smsh = shift_stride;
  p.scale_bias = scale_bias; p.shift_bias = shift_bias;
  p.y = static_cast<uint16_t*>(norm_out); p.sy = norm_out_stride;
  if (!residual)
    return launch_fwd<IN_PLAIN, EPI_LN_MOD_BF16>(p, static_cast<hipStream_t>(stream));
  p.r = static_cast<const uint16_t*>(residual); p.sr = residual_stride;
  p.h = static_cast<uint16_t*>(residual_out); p.sh = residual_out_stride;
  return launch_fwd<IN_ADD, EPI_LN_MOD_BF16>(p, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ RMSNorm + SiLU

dn_status dn_fused_rmsnorm_silu(void* out, int64_t out_stride, int output_fp8,
                                const float* scale, const void* x, int64_t x_stride,
                                const void* w, int w_dtype, float w_bias, int64_t rows,
                                int64_t hidden, float eps, dn_stream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (output_fp8 != 0 && output_fp8 != 1)
    return fail(DN_ERR_DTYPE, "output_fp8 must be 0 or 1");
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, hidden, 2, "x"));
  DN_CHECK(check_matrix(out, out_stride, hidden, output_fp8 ? 1 : 2, "out"));
  DN_CHECK(check_weight(w, w_dtype));
  if (output_fp8) DN_CHECK(check_f32(scale, "scale", true));
  FwdParams p = base_params(rows, hidden, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  if (output_fp8) {
    p.q = static_cast<uint8_t*>(out); p.sq = out_stride;
    p.scale = scale;
    return launch_fwd<IN_PLAIN, EPI_SILU_FP8>(p, static_cast<hipStream_t>(stream));
  }
  p.y = static_cast<uint16_t*>(out); p.sy = out_stride;
  return launch_fwd<IN_PLAIN, EPI_SILU_BF16>(p, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ gated-residual RMSNorm

namespace {

dn_status gres_common(void* next_out, int64_t next_out_stride, void* residual,
                      int64_t residual_stride, const void* branch, int64_t branch_stride,
                      const void* gate, int64_t gate_stride, int64_t gate_rows, const void* w,
                      int w_dtype, float w_bias, const void* w_next, int w_next_dtype,
                      float w_next_bias, int64_t rows, int64_t hidden, float eps, bool next,
                      hipStream_t stream) {
  DN_CHECK(check_shape(rows, hidden, 8, "hidden"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(residual, residual_stride, hidden, 2, "residual"));
  DN_CHECK(check_matrix(branch, branch_stride, hidden, 2, "branch"));
  if (gate_rows != 1 && gate_rows != rows)
    return fail(DN_ERR_SHAPE, "gate_rows must be 1 or rows (%lld), got %lld", (long long)rows,
                (long long)gate_rows);
  DN_CHECK(check_matrix(gate, gate_stride, hidden, 2, "gate"));
  DN_CHECK(check_weight(w, w_dtype));
  if (next) {
    DN_CHECK(check_matrix(next_out, next_out_stride, hidden, 2, "out"));
    DN_CHECK(check_weight(w_next, w_next_dtype));
  }
  GresParams p{};
  p.b = static_cast<const uint16_t*>(branch); p.sb = branch_stride;
  p.r = static_cast<uint16_t*>(residual); p.sr = residual_stride;
  p.g = static_cast<const uint16_t*>(gate); p.sg = gate_stride; p.g_bcast = gate_rows == 1;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  p.w2 = w_next; p.w2_f32 = w_next_dtype == DN_WEIGHT_F32; p.w2_bias = w_next_bias;
  p.y = static_cast<uint16_t*>(next_out); p.sy = next_out_stride;
  p.rows = rows;
  p.hidden = (int)hidden;
  p.nvec = (int)(hidden / 8);
  p.eps = eps;
  p.w_in_lds = p.nvec <= kMaxLdsWeightVectors;
  const int tier = pick_fwd_tier(p.nvec, 6, g_force_tpr.load());
  if (tier < 0) return fail(DN_ERR_SHAPE, "hidden %lld is too wide", (long long)hidden);
  const TierShape s = fwd_tier_shape(tier);
  const int g = s.nt / s.tpr;
  const int wpr = s.tpr > 64 ? s.tpr / 64 : 1;
  const size_t lds = gres_lds_bytes(p.nvec, p.w_in_lds, next, g, wpr, s.r);
  auto launch = [&](int grid, hipStream_t st, const void** k) -> hipError_t {
    return next ? gres_launch<true>(p, tier, grid, lds, st, k)
                : gres_launch<false>(p, tier, grid, lds, st, k);
  };
  const void* kernel = nullptr;
  if (launch(0, nullptr, &kernel) != hipSuccess || !kernel)
    return fail(DN_ERR_HIP, "no kernel instance for tier %d", tier);
  const int64_t per_iter = (int64_t)g * s.r;
  const int64_t needed = (rows + per_iter - 1) / per_iter;
  int grid = 0;
  DN_CHECK(persistent_grid(kernel, s.nt, lds, DN_BLOCKS_PER_CU, needed, &grid));
  const hipError_t e = launch(grid, stream, nullptr);
  if (e != hipSuccess) return fail(DN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return DN_OK;
}

}  // namespace

dn_status dn_gated_residual_rmsnorm(void* residual, int64_t residual_stride,
                                    const void* branch, int64_t branch_stride,
                                    const void* gate, int64_t gate_stride, int64_t gate_rows,
                                    const void* w, int w_dtype, float w_bias, int64_t rows,
                                    int64_t hidden, float eps, dn_stream_t stream) {
  return gres_common(nullptr, 0, residual, residual_stride, branch, branch_stride, gate,
                     gate_stride, gate_rows, w, w_dtype, w_bias, nullptr, 0, 0.0f, rows, hidden,
                     eps, false, static_cast<hipStream_t>(stream));
}

dn_status dn_gated_residual_next_rmsnorm(void* out, int64_t out_stride, void* residual,
                                         int64_t residual_stride, const void* branch,
                                         int64_t branch_stride, const void* gate,
                                         int64_t gate_stride, int64_t gate_rows, const void* w,
                                         int w_dtype, float w_bias, const void* w_next,
                                         int w_next_dtype, float w_next_bias, int64_t rows,
                                         int64_t hidden, float eps, dn_stream_t stream) {
  return gres_common(out, out_stride, residual, residual_stride, branch, branch_stride, gate,
                     gate_stride, gate_rows, w, w_dtype, w_bias, w_next, w_next_dtype,
                     w_next_bias, rows, hidden, eps, true, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ RMSNorm * sigmoid(gate)

dn_status dn_rmsnorm_sigmoid_gate(void* x, int64_t x_stride, const void* gate,
                                  int64_t gate_stride, const void* w, int w_dtype, float w_bias,
                                  int64_t rows, int64_t head_dim, float eps,
                                  dn_stream_t stream) {
  DN_CHECK(check_shape(rows, head_dim, 8, "head_dim"));
  if (rows == 0) return DN_OK;  // empty tensors may carry NULL pointers
  DN_CHECK(check_matrix(x, x_stride, head_dim, 2, "x"));
  DN_CHECK(check_matrix(gate, gate_stride, head_dim, 2, "gate"));
  if (w) DN_CHECK(check_weight(w, w_dtype));
  FwdParams p = base_params(rows, head_dim, eps);
  p.x = static_cast<const uint16_t*>(x); p.sx = x_stride;
  p.y = static_cast<uint16_t*>(x); p.sy = x_stride;
  p.gate = static_cast<const uint16_t*>(gate); p.sg = gate_stride;
  p.w = w; p.w_f32 = w_dtype == DN_WEIGHT_F32; p.w_bias = w_bias;
  return launch_fwd<IN_PLAIN, EPI_SIGMOID_GATE>(p, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ fused QK norm + RoPE

dn_status dn_fused_qk_rmsnorm_rope(
    void* q_out, int64_t q_out_stride, void* k_out, int64_t k_out_stride, void* v_out,
    int64_t v_out_stride, int output_fp8, const float* output_quant_scale,
    const float* v_quant_scale, const void* qkv, int64_t qkv_stride, const void* q_weight,
    const void* k_weight, int w_dtype, int is_qk_norm, int64_t tokens, int num_heads_q,
    int num_heads_k, int num_heads_v, int head_dim, int ppf, int pph, int ppw,
    int num_frame_channels, int num_height_channels, int num_width_channels, double base,
    int interleave, double yarn_factor, double yarn_low, double yarn_high,
    float attention_factor, float eps, dn_stream_t stream) {
  if (tokens < 0) return fail(DN_ERR_SHAPE, "tokens must be >= 0 (got %lld)", (long long)tokens);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(DN_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256 (got %d)", head_dim);
  if (num_heads_q < 1 || num_heads_k < 1 || num_heads_v < 1 || num_heads_q > 32 ||
      num_heads_k > 32 || num_heads_v > 32)
    return fail(DN_ERR_SHAPE, "head counts must be in [1, 32] (got %d, %d, %d)", num_heads_q,
                num_heads_k, num_heads_v);
  const int cf = num_frame_channels, ch = num_height_channels, cw = num_width_channels;
  if (cf < 0 || ch < 0 || cw < 0 || cf % 2 || ch % 2 || cw % 2 || cf + ch + cw != head_dim)
    return fail(DN_ERR_SHAPE,
                "frame/height/width channels must be even, >= 0 and sum to head_dim %d "
                "(got %d, %d, %d)", head_dim, cf, ch, cw);
  if (ppf < 1 || pph < 1 || ppw < 1)
    return fail(DN_ERR_SHAPE, "ppf, pph and ppw must be >= 1");
  const int64_t seq = (int64_t)ppf * pph * ppw;
  if (tokens >= ((int64_t)1 << 31) || seq >= ((int64_t)1 << 31))
    return fail(DN_ERR_SHAPE, "tokens and ppf*pph*ppw must stay below 2^31");
  if (tokens % seq != 0)
    return fail(DN_ERR_SHAPE, "tokens %lld is not a multiple of ppf*pph*ppw = %lld",
                (long long)tokens, (long long)seq);
  if (!(base > 0.0)) return fail(DN_ERR_SHAPE, "base must be > 0");
  if (!(yarn_factor > 0.0)) return fail(DN_ERR_SHAPE, "yarn factor must be > 0");
  if (yarn_factor == 1.0 && attention_factor != 1.0f)
    return fail(DN_ERR_SHAPE, "attention_factor must be 1.0 when the yarn factor is 1.0");
  if (output_fp8 != 0 && output_fp8 != 1)
    return fail(DN_ERR_DTYPE, "output_fp8 must be 0 or 1");
  if (tokens == 0) return DN_OK;  // empty tensors may carry NULL pointers
  const int width = (num_heads_q + num_heads_k + num_heads_v) * head_dim;
  DN_CHECK(check_matrix(qkv, qkv_stride, width, 2, "qkv"));
  const int oe = output_fp8 ? 1 : 2;
  DN_CHECK(check_matrix(q_out, q_out_stride, (int64_t)num_heads_q * head_dim, oe, "q_out"));
  DN_CHECK(check_matrix(k_out, k_out_stride, (int64_t)num_heads_k * head_dim, oe, "k_out"));
  DN_CHECK(check_matrix(v_out, v_out_stride, (int64_t)num_heads_v * head_dim, oe, "v_out"));
  if (is_qk_norm) {
    DN_CHECK(check_weight(q_weight, w_dtype));
    if (!k_weight) return fail(DN_ERR_NULL, "k_weight must not be NULL");
    if (!aligned(k_weight, 16)) return fail(DN_ERR_ALIGN, "k_weight must be 16-byte aligned");
  }
  if (output_fp8) {
    DN_CHECK(check_f32(output_quant_scale, "output_quant_scale", true));
    DN_CHECK(check_f32(v_quant_scale, "v_quant_scale", true));
  }
  RopeParams p{};
  p.qkv = static_cast<const uint16_t*>(qkv); p.sqkv = qkv_stride;
  p.wq = q_weight; p.wk = k_weight; p.w_f32 = w_dtype == DN_WEIGHT_F32;
  p.qo = q_out; p.sqo = q_out_stride;
  p.ko = k_out; p.sko = k_out_stride;
  p.vo = v_out; p.svo = v_out_stride;
  p.qk_scale = output_quant_scale; p.v_scale = v_quant_scale;
  p.rows = tokens;
  p.nq = num_heads_q; p.nk = num_heads_k; p.nv = num_heads_v; p.hd = head_dim;
  p.cf = cf; p.ch = ch; p.cw = cw;
  p.ppf = ppf; p.pph = pph; p.ppw = ppw;
  p.eps = eps; p.af = attention_factor;
  p.base = base; p.factor = yarn_factor; p.low = yarn_low; p.high = yarn_high;
  p.qk_norm = is_qk_norm != 0;
  p.nvec = width / 8;
  p.nwvec = (num_heads_q + num_heads_k) * head_dim / 8;
  p.w_in_lds = p.qk_norm && p.nwvec <= kMaxLdsWeightVectors;

  const bool neox = interleave == 0;
  const int units = neox ? p.nvec / 2 : p.nvec;
  int tier = -1;
  for (int t = 0; t < kRopeTierCount && tier < 0; ++t) {
    const TierShape ts = rope_tier_shape(t);
    if (ts.tpr * (neox ? ts.vmax / 2 : ts.vmax) >= units) tier = t;
  }
  if (tier < 0) return fail(DN_ERR_SHAPE, "the qkv row is too wide");
  const TierShape ts = rope_tier_shape(tier);
  const int g = ts.nt / ts.tpr;
  const int wpr = ts.tpr > 64 ? ts.tpr / 64 : 1;
  const size_t lds = rope_lds_bytes(p.w_in_lds, p.nwvec, head_dim, g, wpr);
  auto launch = [&](int grid, hipStream_t st, const void** k) -> hipError_t {
    if (neox)
      return output_fp8 ? rope_launch<true, true>(p, tier, grid, lds, st, k)
                        : rope_launch<true, false>(p, tier, grid, lds, st, k);
    return output_fp8 ? rope_launch<false, true>(p, tier, grid, lds, st, k)
                      : rope_launch<false, false>(p, tier, grid, lds, st, k);
  };
  const void* kernel = nullptr;
  if (launch(0, nullptr, &kernel) != hipSuccess || !kernel)
    return fail(DN_ERR_HIP, "no kernel instance for rope tier %d", tier);
  const int64_t needed = (tokens + g - 1) / g;
  int grid = 0;
  DN_CHECK(persistent_grid(kernel, ts.nt, lds, DN_BLOCKS_PER_CU_SINGLE, needed, &grid));
  const hipError_t e = launch(grid, static_cast<hipStream_t>(stream), nullptr);
  if (e != hipSuccess) return fail(DN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return DN_OK;
}

}  // extern "C"
