/*
 * dnorm.h -- C ABI of the row-wise RMSNorm and LayerNorm families on AMD Instinct MI355X
 * (gfx950).
 *
 * Every operation normalises rows of a [rows, hidden] matrix independently.  RMSNorm:
 *
 *     r_t  = 1 / sqrt(mean_j h_tj^2 + eps)        (FP32 statistics, eps an FP32 number)
 *     y_tj = BF16((h_tj * r_t) * w_eff_j),  w_eff_j = FP32(w_j + w_bias)
 *
 * LayerNorm (population variance over the row):
 *
 *     m_t  = mean_j h_tj,  r_t = 1 / sqrt(mean_j (h_tj - m_t)^2 + eps)
 *     n_tj = (h_tj - m_t) * r_t,  y_tj = n_tj * gamma_j + beta_j
 *
 * Pages cited (by title and section):
 *   [norm docs]   "flashinfer.norm" API reference: the API table and the section
 *                 "Training RMSNorm (Cake)".
 *   [norm guide]  "FlashInfer 归一化算子库全解 ..." walk-through article, by section number.
 *   [cake docs]   "flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_forward":
 *                 Parameters, Returns, Notes.
 *   [flashrt]     "flashrt-adaptive-norms" README: Exported APIs, Tensor Conventions.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers on the current HIP device.  Matrices are
 *     row-major with an explicit row stride counted in ELEMENTS (>= hidden); the feature
 *     dimension is contiguous.  A 3-D [T, heads, hd] tensor whose leading dimensions are
 *     contiguous with one another is passed as rows = T*heads, hidden = hd ([norm guide]
 *     §2.1: 3-D input is normalised per (batch, head) row; [cake docs] Parameters: x).
 *   - BF16 and FP32 tensors need 16-byte aligned bases and row strides that are multiples
 *     of 8 elements; FP8 outputs need 8-byte aligned bases and strides that are multiples
 *     of 8; per-row FP32 vectors (rstd, block scales, dw) need 4-byte alignment.  Row
 *     strides are at most 2^24 elements.
 *   - hidden must be a positive multiple of 8 and at most dn_max_hidden().
 *   - rows == 0 is valid: once rows and hidden pass their checks the call returns DN_OK
 *     and launches nothing; pointers may then be NULL ([norm guide] §6.1).
 *   - Outputs are caller-owned and preallocated (destination passing, [norm guide] §2.1).
 *     An output may alias an input exactly (same pointer, same stride) -- that is how the
 *     in-place calls work -- but must not overlap it in any other way.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).  The
 *     library never allocates device memory and never synchronises; FP8 scales are read
 *     from device memory, so no host round trip happens.
 *   - Errors: every argument check runs on the host before anything is launched.  A failed
 *     check returns a negative dn_status, records a message for dn_last_error(), and
 *     launches nothing.  DN_ERR_HIP reports a failed HIP call or launch.
 *   - Rounding: round-to-nearest-even for BF16, FP32 and FP8.  FP8 is OCP e4m3fn; values
 *     beyond +-448 saturate to +-448.  NaN or infinite inputs give unspecified outputs.
 */
#ifndef DNORM_H
#define DNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* dn_stream_t; /* hipStream_t */

typedef enum dn_status {
  DN_OK = 0,
  DN_ERR_NULL = -1,        /* a required pointer is NULL */
  DN_ERR_SHAPE = -2,       /* negative rows, hidden out of range, stride < hidden, ... */
  DN_ERR_ALIGN = -3,       /* a pointer or stride breaks the alignment rules above */
  DN_ERR_DTYPE = -4,       /* unknown weight dtype code */
  DN_ERR_WORKSPACE = -5,   /* backward workspace too small or not 256-byte aligned */
  DN_ERR_UNSUPPORTED = -6, /* hidden not a multiple of 8 (or of 128 for 1x128 blocks) */
  DN_ERR_HIP = -7          /* a HIP runtime call or kernel launch failed */
} dn_status;

/* Weight dtypes: BF16 [hidden], or FP32 [hidden] (a zero-centred weight whose effective
 * value 1 + w is formed in FP32 with w_bias = 1; [cake docs] Parameters: w). */
enum { DN_WEIGHT_BF16 = 0, DN_WEIGHT_F32 = 1 };

/* Message of the last failed call made on this host thread ("" if none). */
const char* dn_last_error(void);

/* Largest supported hidden size (32768). */
int dn_max_hidden(void);

/* Library version string. */
const char* dn_version(void);

/* ---------------------------------------------------------------------------------------
 * rmsnorm / gemma_rmsnorm   ([norm docs] API table; [norm guide] §2.1, §2.2)
 *   y = BF16(x * r * FP32(w + w_bias)); rstd[t] = FP32(r_t) when rstd != NULL.
 *   w_bias = 0 is rmsnorm, w_bias = 1 the Gemma form (w + 1).
 *   x: BF16 [rows, hidden] (stride x_stride); w: [hidden] of dtype w_dtype;
 *   y: BF16 [rows, hidden] (stride y_stride; may be x itself); rstd: FP32 [rows] or NULL.
 */
dn_status dn_rmsnorm(void* y, int64_t y_stride, float* rstd,
                     const void* x, int64_t x_stride,
                     const void* w, int w_dtype, float w_bias,
                     int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * rmsnorm_quant   ([norm docs] API table: rmsnorm_quant(out, input, weight, scale))
 *   out = e4m3fn((x * r * w_eff) / scale), from the unrounded FP32 normalised value.
 *   scale: device FP32 [1] ([norm guide] §3.2).  out: FP8 [rows, hidden] (stride out_stride).
 */
dn_status dn_rmsnorm_quant(uint8_t* out, int64_t out_stride,
                           const void* x, int64_t x_stride,
                           const void* w, int w_dtype, float w_bias, const float* scale,
                           int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * fused_add_rmsnorm / gemma_fused_add_rmsnorm   ([norm docs] API table; [norm guide] §3.1)
 *   In place: residual <- h_new = BF16(x + residual); x <- BF16(h_new * r * w_eff).
 *   The norm is taken over the BF16 h_new ([cake docs] Parameters: x).
 *   rstd: FP32 [rows] or NULL.
 */
dn_status dn_fused_add_rmsnorm(void* x, int64_t x_stride,
                               void* residual, int64_t residual_stride,
                               const void* w, int w_dtype, float w_bias, float* rstd,
                               int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * fused_add_rmsnorm_quant   ([norm docs] API table; [norm guide] §3.2)
 *   residual <- h_new = BF16(x + residual); out = e4m3fn((h_new * r * w_eff) / scale).
 *   x is read only.  scale: device FP32 [1].
 */
dn_status dn_fused_add_rmsnorm_quant(uint8_t* out, int64_t out_stride,
                                     const void* x, int64_t x_stride,
                                     void* residual, int64_t residual_stride,
                                     const void* w, int w_dtype, float w_bias,
                                     const float* scale,
                                     int64_t rows, int64_t hidden, float eps,
                                     dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * fused_add_rmsnorm_fp8_block_quant   ([norm docs] API table; [norm guide] §3.3)
 *   One pass: residual <- h_new = BF16(x + residual); n = BF16(h_new * r * w_eff);
 *   for each 1x128 block k of a row: s = FP32(max|n| / 448), out = e4m3fn(n / s)
 *   (s = 0 and out = 0 for an all-zero block).
 *   block_scale: FP32, column-major "MN-major" [hidden/128][scale_ld]: the scale of row t,
 *   block k is block_scale[k * scale_ld + t]; scale_ld >= rows (the pages use
 *   round_up(rows, 4)); entries t in [rows, scale_ld) are written as 0.
 *   normed_out: BF16 [rows, hidden] receiving n, or NULL.  hidden % 128 == 0.
 */
dn_status dn_fused_add_rmsnorm_fp8_block_quant(uint8_t* out, int64_t out_stride,
                                               float* block_scale, int64_t scale_ld,
                                               void* normed_out, int64_t normed_stride,
                                               const void* x, int64_t x_stride,
                                               void* residual, int64_t residual_stride,
                                               const void* w, int w_dtype, float w_bias,
                                               int64_t rows, int64_t hidden, float eps,
                                               dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * ada_rms_norm   ([flashrt] Exported APIs: ada_rms_norm_style_bf16; Tensor Conventions)
 *   n = x * r * w (BF16 weight, no bias); out = BF16(n * (1 + style_scale) + style_shift);
 *   gate_out = the style's third chunk (a bit copy).
 *   style: BF16 [style_rows, 3*dim] with chunks [scale | shift | gate]; style_rows is
 *   rows (one style row per token) or 1 (one row broadcast to every token).
 *   gate_out: BF16 [rows, dim] or NULL.  Every rows x dim matrix has its own stride.
 */
dn_status dn_ada_rms_norm(void* out, int64_t out_stride,
                          void* gate_out, int64_t gate_out_stride,
                          const void* x, int64_t x_stride,
                          const void* w,
                          const void* style, int64_t style_stride, int64_t style_rows,
                          int64_t rows, int64_t dim, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * gate_residual_ada_norm_fp8   ([flashrt] Exported APIs:
 *                                gate_residual_ada_norm_fp8_static_bf16)
 *   residual <- h = BF16(FP32-FMA(x, gate, residual));
 *   out = e4m3fn((h * r * w * (1 + style_scale) + style_shift) / scale);
 *   gate_out = the style's third chunk.  scale: device FP32 [1].
 */
dn_status dn_gate_residual_ada_norm_fp8(void* residual, int64_t residual_stride,
                                        uint8_t* out, int64_t out_stride,
                                        void* gate_out, int64_t gate_out_stride,
                                        const void* x, int64_t x_stride,
                                        const void* gate, int64_t gate_stride,
                                        const void* w,
                                        const void* style, int64_t style_stride,
                                        int64_t style_rows, const float* scale,
                                        int64_t rows, int64_t dim, float eps,
                                        dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * train_forward   ([norm docs] "Training RMSNorm (Cake)": cake_rmsnorm_train_forward;
 *                  [cake docs] Parameters, Returns; [norm guide] §6.1, §6.2)
 *   Without residual: y = BF16(x * r * w_eff), rstd = FP32(r).
 *   With residual (non-NULL): h_new = BF16(x + residual) is written to h_new and is the
 *   normalised value.  rstd (FP32 [rows]) is required: it is what the backward needs.
 *   w: BF16, or FP32 with w_bias = 1 for the zero-centred form.
 */
dn_status dn_train_forward(void* y, int64_t y_stride, float* rstd,
                           void* h_new, int64_t h_new_stride,
                           const void* x, int64_t x_stride,
                           const void* residual, int64_t residual_stride,
                           const void* w, int w_dtype, float w_bias,
                           int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Training backward   ([norm docs] cake_rmsnorm_train_backward, ..._workspace_bytes;
 *                      [norm guide] §6.1-6.4)
 *   dx = BF16(r*g*w_eff - x*r^3*mean_j(g*w_eff*x) [+ g_residual]), evaluated in FP32 as
 *        r*(g*w_eff - x*(r^2*mean)) so that the coefficient stays in FP32's range for rows
 *        whose scale is far from 1 (mean_j and r^2*mean in FP64)
 *   Range: the products g*x (the row's dot product and dw's terms) are formed in FP32, so
 *   the stated accuracy needs |g|*|x| inside FP32's normal range (about 1e-38 .. 3e38);
 *   beyond it dx and dw lose accuracy (dw stays bitwise deterministic).
 *   dw = FP32(sum_t g*x*r)     -- the gradient with respect to w_eff (= w + w_bias)
 *   x is the tensor the forward normalised (h_new on the residual route) and rstd the FP32
 *   tensor the forward returned.  g_residual (nullable) is the gradient reaching h_new
 *   directly; dx is then the gradient of both residual inputs.
 *   dw_dtype: DN_WEIGHT_F32 writes FP32 dw [hidden]; DN_WEIGHT_BF16 writes BF16 dw
 *   [hidden], the FP32 value rounded once more ([norm guide] §6.4: dw is accumulated in
 *   FP32 and cast to the weight's dtype).
 *
 *   dw is bitwise deterministic: rows are cut into min(rows, 256) fixed chunks that depend
 *   on rows only (not on the device); each chunk's column sums are carried in FP64 from
 *   exact products into one workspace row, and a second launch on the same stream adds the
 *   chunk rows in a fixed order (eight contiguous ranges of chunks, each in chunk order,
 *   then the ranges in order) before one rounding to FP32.
 *
 *   workspace: caller-owned device memory of at least
 *   dn_train_backward_workspace_bytes(hidden) = 256 * hidden * 8 bytes (FP64 chunk rows),
 *   256-byte aligned.  It needs no zeroing: every call rewrites the chunk rows it reads, so
 *   one buffer serves every call, token count and stream-ordered replay.  Calls sharing a
 *   workspace must be stream-ordered.  (The pages' workspace-size call also takes a
 *   residual flag; the size here depends on neither it nor rows, so only hidden is passed.)
 */
size_t dn_train_backward_workspace_bytes(int64_t hidden);

dn_status dn_train_backward(void* dx, int64_t dx_stride, void* dw, int dw_dtype,
                            const void* g, int64_t g_stride,
                            const void* x, int64_t x_stride,
                            const void* w, int w_dtype, float w_bias, const float* rstd,
                            const void* g_residual, int64_t g_residual_stride,
                            void* workspace, size_t workspace_bytes,
                            int64_t rows, int64_t hidden, dn_stream_t stream);

/* dn_train_backward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and bits as dn_train_backward, for hidden up to 8192
 * (DN_ERR_UNSUPPORTED beyond).  The chunk rows live in a static device array of the
 * library (16 MiB per GPU, held until the process ends; nothing in it needs clearing); the
 * first call on a device looks its address up.  The call allocates nothing.  Every call on
 * one GPU shares that array: calls that overlap on one GPU (different streams without
 * ordering, or several host threads) race and give wrong dw; stream-ordered calls are
 * safe. */
dn_status dn_train_backward_noalloc(void* dx, int64_t dx_stride, void* dw, int dw_dtype,
                                    const void* g, int64_t g_stride,
                                    const void* x, int64_t x_stride,
                                    const void* w, int w_dtype, float w_bias,
                                    const float* rstd,
                                    const void* g_residual, int64_t g_residual_stride,
                                    int64_t rows, int64_t hidden, dn_stream_t stream);

/* The two launches of dn_train_backward, exposed so a caller can place the dw reduction
 * elsewhere (e.g. after exchanging chunk rows between data-parallel ranks) or time them
 * apart.  partials followed by reduce on the same stream is dn_train_backward.
 *   partials: dx, and the FP64 per-chunk column sums in the workspace.
 *   reduce:   dw[j] = the fixed-order sum of the chunk rows of column j, rounded to FP32
 *             (and to BF16 for DN_WEIGHT_BF16); `rows` must equal the rows given to the
 *             partials call (it fixes the chunk count). */
dn_status dn_train_backward_partials(void* dx, int64_t dx_stride,
                                     const void* g, int64_t g_stride,
                                     const void* x, int64_t x_stride,
                                     const void* w, int w_dtype, float w_bias,
                                     const float* rstd,
                                     const void* g_residual, int64_t g_residual_stride,
                                     void* workspace, size_t workspace_bytes,
                                     int64_t rows, int64_t hidden, dn_stream_t stream);

dn_status dn_train_backward_reduce(void* dw, int dw_dtype, const void* workspace,
                                   size_t workspace_bytes, int64_t rows, int64_t hidden,
                                   dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * LayerNorm family   ([norm docs] API table: layernorm, layernorm_quant and the three
 *                     fused_dit_* calls; [norm guide] §4, §5.3)
 *
 * Statistics: the row's sum and sum of squares are accumulated in FP64 from the BF16
 * values (exactly converted), mean = sum/hidden and variance = sum of squares/hidden -
 * mean^2 in FP64 (clamped at 0), r = 1/sqrt(variance + eps) in FP64; mean and r are then
 * rounded once to FP32 and n = (h - mean) * r is evaluated in FP32.
 *
 * layernorm:        y = BF16(FMA(n, gamma, beta)).
 * layernorm_quant:  out = e4m3fn(FMA(n, gamma, beta) / scale); scale: device FP32 [1]
 *                   (applied as a multiplication by its FP32 reciprocal).
 *   x: BF16 [rows, hidden]; gamma, beta: FP32 [hidden], 16-byte aligned, required.
 */
dn_status dn_layernorm(void* y, int64_t y_stride, const void* x, int64_t x_stride,
                       const float* gamma, const float* beta,
                       int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

dn_status dn_layernorm_quant(uint8_t* out, int64_t out_stride,
                             const void* x, int64_t x_stride,
                             const float* gamma, const float* beta, const float* scale,
                             int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

/* DiT gate/residual + LayerNorm, the three modes of [norm guide] §5.3 (BF16 outputs):
 *
 *   gate_residual + gamma/beta:
 *     residual_out = BF16(FP32-FMA(x, FP32(gate + gate_bias), residual))
 *     norm_out     = BF16(FMA(n(residual_out), gamma, beta))
 *   gate_residual + scale/shift:
 *     residual_out as above;
 *     norm_out = BF16(FMA(n(residual_out), FP32(FP32(1 + scale) + scale_bias),
 *                         FP32(shift + shift_bias)))
 *   residual + scale/shift:
 *     h = BF16(x + residual) (written to residual_out when given), or h = x when
 *     residual is NULL (residual_out must then be NULL too); norm_out as in the
 *     scale/shift mode with n(h).
 *
 *   x, residual: BF16 [rows, hidden].  gate, scale, shift: BF16 [rows, hidden] with their
 *   own row strides, so the per-token chunks of one modulation tensor (row stride
 *   6*hidden, [norm guide] §5.3) are passed without a copy.  gate_bias, scale_bias and
 *   shift_bias are FP32 scalars.  residual_out is optional (NULL: not written) and may be
 *   residual itself (in place); norm_out is required.  Any hidden that is a multiple of 8
 *   is accepted (the pages' DiT model uses 3072).
 */
dn_status dn_fused_dit_gate_residual_layernorm_gamma_beta(
    void* residual_out, int64_t residual_out_stride, void* norm_out, int64_t norm_out_stride,
    const void* x, int64_t x_stride, const void* residual, int64_t residual_stride,
    const void* gate, int64_t gate_stride, float gate_bias,
    const float* gamma, const float* beta,
    int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

dn_status dn_fused_dit_gate_residual_layernorm_scale_shift(
    void* residual_out, int64_t residual_out_stride, void* norm_out, int64_t norm_out_stride,
    const void* x, int64_t x_stride, const void* residual, int64_t residual_stride,
    const void* gate, int64_t gate_stride, float gate_bias,
    const void* scale, int64_t scale_stride, float scale_bias,
    const void* shift, int64_t shift_stride, float shift_bias,
    int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

dn_status dn_fused_dit_residual_layernorm_scale_shift(
    void* residual_out, int64_t residual_out_stride, void* norm_out, int64_t norm_out_stride,
    const void* x, int64_t x_stride, const void* residual, int64_t residual_stride,
    const void* scale, int64_t scale_stride, float scale_bias,
    const void* shift, int64_t shift_stride, float shift_bias,
    int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * fused_rmsnorm_silu   ([norm docs] API table: fused_rmsnorm_silu; [norm guide] §5.1)
 *   y = (x * r) * FP32(w + w_bias) as rmsnorm (unrounded), s = y / (1 + exp(-y)) in FP32:
 *   (y or y*e) * (1/(1 + e)) with e = exp(-|y|) (no overflow) on the hardware exp2 and
 *   reciprocal, within (|y| + 5) FP32 ulps of the exact SiLU of y.
 *   output_fp8 == 0: out BF16 [rows, hidden] = BF16(s).
 *   output_fp8 == 1: out e4m3fn [rows, hidden] = e4m3fn(s / *scale), scale a device FP32
 *   [1] (the pages leave the FP8 scale open; pass 1.0 for a plain conversion).
 *   The pages' NVFP4 output and the engine workspace of their implementation have no
 *   counterpart here (no workspace is needed).
 */
dn_status dn_fused_rmsnorm_silu(void* out, int64_t out_stride, int output_fp8,
                                const float* scale, const void* x, int64_t x_stride,
                                const void* w, int w_dtype, float w_bias,
                                int64_t rows, int64_t hidden, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * gated_residual_rmsnorm / gated_residual_next_rmsnorm
 *   ([norm docs] Fixed-Width Fused Norms: a normalised branch is blended into the
 *    residual stream; the second call also normalises the result for the next layer, in
 *    the same launch)
 *   The pages give no formula; the reading implemented:
 *     n = (branch * r_b) * FP32(w + w_bias)            (rmsnorm of the branch, unrounded)
 *     residual <- h = BF16(FMA(gate, n, residual))     (one FP32 rounding, then BF16)
 *     next only: out = BF16((h * r_h) * FP32(w_next + w_next_bias)), r_h the rstd of the
 *                BF16 row h (normalised in the same launch).
 *   gate: BF16 [gate_rows, hidden], gate_rows = rows (one gate row per token) or 1 (one row
 *   shared by every token, e.g. a per-channel gate).  Any hidden that is a multiple of 8
 *   is accepted (the pages' kernels take 8192 only).
 */
dn_status dn_gated_residual_rmsnorm(void* residual, int64_t residual_stride,
                                    const void* branch, int64_t branch_stride,
                                    const void* gate, int64_t gate_stride, int64_t gate_rows,
                                    const void* w, int w_dtype, float w_bias,
                                    int64_t rows, int64_t hidden, float eps,
                                    dn_stream_t stream);

dn_status dn_gated_residual_next_rmsnorm(void* out, int64_t out_stride,
                                         void* residual, int64_t residual_stride,
                                         const void* branch, int64_t branch_stride,
                                         const void* gate, int64_t gate_stride,
                                         int64_t gate_rows,
                                         const void* w, int w_dtype, float w_bias,
                                         const void* w_next, int w_next_dtype,
                                         float w_next_bias, int64_t rows, int64_t hidden,
                                         float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * rmsnorm_sigmoid_gate   ([norm docs] Fixed-Width Fused Norms: rmsnorm_sigmoid_gate)
 *   The pages name only a per-head RMSNorm followed by a sigmoid gate, done in place, at
 *   head dim 64;
 *   the reading implemented: rows are heads (a [tokens, heads, head_dim] tensor passed as
 *   rows = tokens*heads), y = (x * r) * FP32(w + w_bias) as rmsnorm, then
 *   x <- BF16(y * sigmoid(gate)), gate BF16 of x's shape (own row stride).  w: BF16 or FP32
 *   [head_dim], or NULL for ones.  sigmoid(g) = (1 or e) * 1/(1 + e), e = exp(-|g|), on the
 *   hardware exp2 and reciprocal (within (|g| + 5) FP32 ulps).  Any head_dim that is a
 *   multiple of 8 is accepted (the pages' kernel takes 64 only).
 */
dn_status dn_rmsnorm_sigmoid_gate(void* x, int64_t x_stride, const void* gate,
                                  int64_t gate_stride, const void* w, int w_dtype,
                                  float w_bias, int64_t rows, int64_t head_dim, float eps,
                                  dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * fused_qk_rmsnorm_rope   ([norm docs] API table: fused_qk_rmsnorm_rope; [norm guide] §5.2)
 *
 * qkv: BF16 [tokens, (nq + nk + nv) * head_dim] (row stride qkv_stride), heads in the
 * order Q, K, V.  Per token:
 *   Q and K (is_qk_norm != 0): n = (x * r) * w, r = 1/sqrt(mean(x^2) + eps) taken across
 *     all heads of Q (resp. K); q_weight [nq*head_dim], k_weight [nk*head_dim], BF16 or
 *     FP32 (w_dtype).  is_qk_norm == 0: n = x, weights unused (may be NULL).
 *   3-D rotary embedding of every head: the token's index t in its sequence (t mod
 *     ppf*pph*ppw) gives frame t / (pph*ppw), height (t / ppw) % pph, width t % ppw.
 *     Pair j < head_dim/2 is channels (2j, 2j+1) when interleave != 0, (j, j + head_dim/2)
 *     otherwise (NeoX); the first num_frame_channels/2 pairs turn with the frame, the next
 *     num_height_channels/2 with the height, the rest with the width, at angle
 *     position * inv_freq, inv_freq = base^(-2i/count) for pair i of a group of count
 *     channels.  yarn_factor != 1 blends inv_freq / factor and inv_freq with
 *     ramp = clamp((i - yarn_low) / (yarn_high - yarn_low), 0, 1) (yarn_high == yarn_low
 *     takes yarn_high + 0.001).  (a, b) -> (a cos - b sin, a sin + b cos), with cos and
 *     sin times attention_factor.  Angles are formed and reduced modulo 2*pi in FP64; their
 *     sine and cosine are evaluated in FP32 on the reduced argument.
 *   V: copied bit for bit.
 * Outputs q_out [tokens, nq*head_dim], k_out, v_out (each with its row stride): BF16
 * (output_fp8 == 0; one rounding of the FP32 result), or e4m3fn (output_fp8 == 1): Q and K
 * divided by *output_quant_scale, V by *v_quant_scale (device FP32 [1] each).
 *
 * Limits (the pages'): head_dim in {64, 128, 256}; 1..32 heads of each kind; channel
 * counts even (0 allowed) summing to head_dim; tokens a multiple of ppf*pph*ppw;
 * attention_factor must be 1 when yarn_factor is 1.
 */
dn_status dn_fused_qk_rmsnorm_rope(
    void* q_out, int64_t q_out_stride, void* k_out, int64_t k_out_stride,
    void* v_out, int64_t v_out_stride, int output_fp8,
    const float* output_quant_scale, const float* v_quant_scale,
    const void* qkv, int64_t qkv_stride,
    const void* q_weight, const void* k_weight, int w_dtype, int is_qk_norm,
    int64_t tokens, int num_heads_q, int num_heads_k, int num_heads_v, int head_dim,
    int ppf, int pph, int ppw,
    int num_frame_channels, int num_height_channels, int num_width_channels,
    double base, int interleave, double yarn_factor, double yarn_low, double yarn_high,
    float attention_factor, float eps, dn_stream_t stream);

/* ---------------------------------------------------------------------------------------
 * Test and tuning hook: force the threads that share one row (8, 16, 32, 64, 128, 256,
 * 320, 448, 512 or 1024) in every forward launch of this process; 0 restores the automatic choice
 * by hidden size.  Returns DN_ERR_SHAPE for other values or when the forced count cannot
 * cover hidden in registers (then the automatic choice is used).  Results stay within
 * the documented tolerances either way; bits may change with the row mapping.
 */
dn_status dn_force_threads_per_row(int threads);

#ifdef __cplusplus
}
#endif

#endif /* DNORM_H */
