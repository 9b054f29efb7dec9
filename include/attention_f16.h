/*
 * attention_f16.h -- C ABI of the MI355X (gfx950) fused attention and row
 * softmax kernels.
 *
 *   O = softmax(scale * Q K^T [+ causal mask]) V        (per batch item, head)
 *   Y = softmax(X) along each row
 *
 * Pages this interface follows (titles as printed on them):
 *   [OPS]     CUDA operator practice page (Softmax and GEMM): §2.1 the softmax
 *             of a row (maximum, sum of exp(x - max), division); §2.2 its
 *             online form, which keeps a running maximum m and sum s and
 *             rescales s by exp(m - m') when the maximum grows to m', so a row
 *             is read once; §2.3-§2.4 the row held in registers, or streamed
 *             twice for long rows; §2.5 a row whose elements are all masked
 *             has no finite maximum.
 *   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM
 *             kernel): §1.1 attention is Q K^T, a softmax, then a product with V.
 *   [CATLASS] CATLASS template library page: §5.2 fuses the two products and
 *             the softmax into one kernel so the score matrix never goes to
 *             global memory; §3 keeps matrix products in fp16 with fp32
 *             accumulation and reductions (softmax) in fp32.
 *
 * Attention semantics (indices 0-based, strides in ELEMENTS):
 *   Q(b,h,i,d) = Q[b*q_strides[0] + h*q_strides[1] + i*q_strides[2] + d]
 *   K(b,h,j,d), V(b,h,j,c), O(b,h,i,c) likewise with their own strides;
 *   i < Sq, j < Sk, d, c < D.  Q, K, V are binary16; O is binary16 or fp32.
 *   s_ij = scale * sum_d Q(i,d) K(j,d)             (fp16 products, fp32 sums)
 *   key j is visible to query i unless causal and j > i + (Sk - Sq)
 *   P_ij = exp(s_ij - m_i) / sum_{visible k} exp(s_ik - m_i)   over visible j
 *          (m_i the row's largest visible score; fp32)
 *   O(i,c) = sum_{visible j} P_ij V(j,c)           (P rounded to binary16 for
 *                                                   the product, fp32 sums)
 *   A row with no visible key (causal with i + Sk - Sq < 0, or Sk == 0) is
 *   written as zeros: [OPS] §2.5 notes that the plain formula divides 0 by 0
 *   there and suggests a constant output; zero is the constant taken.
 *   The result is rounded once to binary16 (nearest even) for a binary16 O.
 *
 * Ownership: the caller owns Q, K, V, O and the stream; a plan is host memory
 * only (no device allocation, no synchronisation anywhere); runs are
 * asynchronous on the stream and one plan may run on several streams at once.
 * Errors: the status codes of gemm_f16f32.h (GEMM_OK, GEMM_ERR_*);
 * gemm_f16f32_status_string describes them.
 */
#ifndef ATTENTION_F16_H
#define ATTENTION_F16_H

#include <stdint.h>

#include "gemm_f16f32.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_f16_plan_s *attn_f16_plan_t;   /* opaque, host only */

/*
 * Validates an attention problem and chooses its kernel.  No HIP call.
 *   out        receives the plan (NULL on failure).
 *   batch, heads  >= 1; Sq, Sk >= 0 (Sq == 0: a no-op plan).
 *   D          head dimension of Q, K and V (and of O): 64 or 128, else
 *              UNSUPPORTED.
 *   q_strides, k_strides, v_strides, o_strides  three element strides each
 *              (batch, head, row), >= 0, row stride >= D; else INVALID_ARG.
 *              Q, K, V strides must be multiples of 8 (16-byte rows) and each
 *              (batch, head) slice of Q, K or V must span fewer than 2^30
 *              elements; else UNSUPPORTED.
 *   causal     0 or 1 (mask of the semantics above).
 *   out_type   GEMM_OUT_F16 or GEMM_OUT_F32 (element type of O).
 */
int attn_f16_plan(attn_f16_plan_t *out, int64_t batch, int64_t heads, int64_t Sq, int64_t Sk,
                  int64_t D, const int64_t q_strides[3], const int64_t k_strides[3],
                  const int64_t v_strides[3], const int64_t o_strides[3], int causal,
                  int out_type);

/*
 * Runs a plan on `stream` (one kernel launch) and returns without waiting.
 *   Q, K, V  device pointers to binary16 storage, 16-byte aligned (else
 *            INVALID_ARG).
 *   O        device pointer to binary16 or fp32 storage, written; must not
 *            overlap Q, K or V (INVALID_ARG).
 *   scale    fp32 factor on the scores (1/sqrt(D) for the usual attention).
 * NULL plan, Q or O (unless the plan is a no-op), or NULL K or V with Sk > 0
 * -> INVALID_ARG (with Sk == 0 neither K nor V is read); a failed launch ->
 * GEMM_ERR_HIP.
 */
int attn_f16_run(attn_f16_plan_t plan, const void *Q, const void *K, const void *V, void *O,
                 float scale, void *stream);

/* Frees a plan (host memory only).  NULL is a no-op.  Returns GEMM_OK. */
int attn_f16_destroy(attn_f16_plan_t plan);

/* Name of the plan's kernel (owned by the plan), "none" for a no-op plan,
 * "invalid" for NULL.  Diagnostic only. */
const char *attn_f16_plan_kernel(attn_f16_plan_t plan);

/*
 * Row softmax: Y(i, j) = exp(X(i,j) - m_i) / sum_k exp(X(i,k) - m_i), in fp32,
 * one launch on `stream`, asynchronous.
 *   rows, cols  >= 0 (either 0: no-op).
 *   x, ldx      device pointer and row stride (elements, >= cols) of X.
 *   in_type     GEMM_OUT_F16 (binary16 X) or GEMM_OUT_F32 (fp32 X).
 *   y, ldy      device pointer and row stride (>= cols) of Y; Y may be X
 *               itself (same pointer, type and stride), otherwise the two may
 *               not overlap.
 *   out_type    GEMM_OUT_F16 or GEMM_OUT_F32.
 * Elements equal to -inf are masked (weight 0); a row with no element above
 * -inf is written as zeros (the constant output of [OPS] §2.5).  Rows of up
 * to 8192 elements are held in registers (read once); longer rows are read
 * twice, the first pass keeping the online maximum and sum of [OPS] §2.2.
 * Bad arguments -> INVALID_ARG; a failed launch -> GEMM_ERR_HIP.
 */
int attn_softmax_rows(int64_t rows, int64_t cols, const void *x, int64_t ldx, int in_type,
                      void *y, int64_t ldy, int out_type, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTENTION_F16_H */
