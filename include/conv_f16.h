/*
 * conv_f16.h -- C ABI of the MI355X (gfx950) implicit-GEMM convolution.
 *
 *   y = act(alpha * conv2d(x, w) + beta * y + bias)
 *
 * Pages this interface follows (titles as printed on them):
 *   [CATLASS] CATLASS template library page: §5.1 a convolution is a
 *             four-deep loop that becomes a matrix product when input windows
 *             and filters are unrolled (im2col); the implicit form never
 *             materialises the unrolled input -- the GEMM's tile iterator
 *             maps row m to an input position and column n to a filter
 *             position and fetches from the input directly, so the GEMM main
 *             loop (tiling, double buffering, matrix instructions) is reused.
 *   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM
 *             kernel): §1.1 convolution via im2col is a GEMM.
 *
 * Semantics (cross-correlation, as neural networks use it; 0-based):
 *   x: N x H x W x C binary16 (NHWC, dense);  w: K x R x S x C binary16
 *   (KRSC, dense);  y: N x P x Q x K (NPQK, dense), binary16 or fp32, with
 *   P = (H + 2 pad_h - dil_h (R - 1) - 1) / stride_h + 1 and Q likewise.
 *   y[n,p,q,k] <- act( fp32(alpha) * sum_{r,s,c} x[n, p stride_h - pad_h + r dil_h,
 *                                                     q stride_w - pad_w + s dil_w, c]
 *                                             * w[k,r,s,c]
 *                      + fp32(beta) * y[n,p,q,k] + bias[k] )
 *   with input positions outside the image contributing zero; fp16
 *   products, fp32 sums, one rounding of the result.  As a GEMM: M = N P Q
 *   rows (output pixels), K output channels as columns, R S C the reduction;
 *   y is read only when beta != 0.
 *
 * Ownership: the caller owns x, w, y, bias and the stream; a plan is host
 * memory only; runs neither allocate nor synchronise, are asynchronous on
 * their stream and need no workspace.  Status codes are those of
 * gemm_f16f32.h (gemm_f16f32_status_string describes them).
 */
#ifndef CONV_F16_H
#define CONV_F16_H

#include <stdint.h>

#include "gemm_f16f32.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct conv_f16_plan_s *conv_f16_plan_t;   /* opaque, host only */

/*
 * Validates a convolution and chooses its kernel.  No HIP call.
 *   N >= 0 (0: a no-op plan); H, W, C, R, S >= 1; K >= 0 (0: no-op);
 *   stride_h, stride_w, dil_h, dil_w >= 1; pad_h, pad_w >= 0; the dilated
 *   filter must fit the padded input (P, Q >= 1) -- else INVALID_ARG.
 *   out_type  GEMM_OUT_F16 or GEMM_OUT_F32, else INVALID_ARG.
 *   x of 2^31 bytes or more, or N P Q, R S C or K at 2^31 or more ->
 *   UNSUPPORTED (32-bit offsets within the input).
 */
int conv_f16_plan(conv_f16_plan_t *out, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K,
                  int64_t R, int64_t S, int64_t stride_h, int64_t stride_w, int64_t pad_h,
                  int64_t pad_w, int64_t dil_h, int64_t dil_w, int out_type);

/* The output's spatial size P x Q.  NULL arguments -> INVALID_ARG. */
int conv_f16_output_size(conv_f16_plan_t plan, int64_t *P, int64_t *Q);

/*
 * Runs a plan on `stream` (one kernel launch), asynchronously.
 *   x, w   device pointers to binary16 storage (const).
 *   y      device pointer to binary16 or fp32 storage, read when beta != 0,
 *          written; must not overlap x, w or the bias (INVALID_ARG).
 *   alpha, beta  fp32 scalars.
 *   bias   NULL or a device pointer to K fp32 values (4-byte aligned).
 *   activation  GEMM_ACT_NONE, _RELU, _GELU or _SILU (applied last).
 * C a multiple of 8 with 16-byte-aligned x and w takes 16-byte loads of 8
 * channels; any other C or alignment takes element-wise loads (same results
 * up to summation order).  NULL plan or pointers (unless the plan is a
 * no-op), a misaligned bias or an unknown activation -> INVALID_ARG; a failed
 * launch -> GEMM_ERR_HIP.
 */
int conv_f16_run(conv_f16_plan_t plan, const void *x, const void *w, void *y, float alpha,
                 float beta, const float *bias, int activation, void *stream);

/* Frees a plan (host memory only).  NULL is a no-op.  Returns GEMM_OK. */
int conv_f16_destroy(conv_f16_plan_t plan);

/* Name of the plan's kernel (owned by the plan), "none" for a no-op plan,
 * "invalid" for NULL.  Diagnostic only. */
const char *conv_f16_plan_kernel(conv_f16_plan_t plan);

#ifdef __cplusplus
}
#endif

#endif /* CONV_F16_H */
