/*
 * gemm_bf16f32.h -- C ABI of the MI355X (gfx950) GEMM on bfloat16 inputs.
 *
 *   C = alpha * A * B + beta * C
 *
 * The same operation, layouts, rules and kernels as gemm_f16f32.h, with A and
 * B holding bfloat16 values instead of binary16: products accumulated in
 * fp32; C (read when beta != 0, then written) is bfloat16 or fp32.
 *
 * Pages this interface follows (titles as printed on them):
 *   [CATLASS] CATLASS template library page: §3.2 defines bfloat16 -- 1 sign
 *             bit, 8 exponent bits (the exponent range of fp32, largest value
 *             about 3.4e38), 7 fraction bits -- and recommends it for
 *             training, where fp16's range overflows.
 *   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM
 *             kernel): §6 names bfloat16 beside fp16 as a GEMM input format
 *             (wide range, coarse precision); §1.3 and §3.4 fix the problem and
 *             the edge rule exactly as for fp16.
 * Everything gemm_f16f32.h states about semantics, leading dimensions,
 * batches, alignment, repacking, the caller-owned workspace, streams and
 * errors holds here unchanged, with "binary16" read as "bfloat16".  The
 * fp32 result is rounded once to bfloat16 (round to nearest even; overflow
 * to +-inf) for a bfloat16 C.
 *
 * A bfloat16 plan is a gemm_f16f32_plan_t made by gemm_bf16f32_plan.  It is
 * run with gemm_bf16f32_run and freed with gemm_f16f32_destroy;
 * gemm_f16f32_workspace_size, gemm_f16f32_workspace_init,
 * gemm_f16f32_plan_kernel and gemm_f16f32_status_string serve both kinds of
 * plan (kernel names of bfloat16 plans start "gemm_bf16_").  Passing a plan
 * to the run function of the other input type -> GEMM_ERR_INVALID_ARG.
 */
#ifndef GEMM_BF16F32_H
#define GEMM_BF16F32_H

#include <stdint.h>

#include "gemm_f16f32.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { GEMM_OUT_BF16 = 2 };   /* element type of C: bfloat16 */

/*
 * Validates a problem with bfloat16 A and B and chooses its kernel.  No
 * device work and no HIP call.  Arguments and rules as gemm_f16f32_plan,
 * except:
 *   out_type  GEMM_OUT_BF16 or GEMM_OUT_F32, else INVALID_ARG
 *             (GEMM_OUT_F16 is not a type of this family).
 */
int gemm_bf16f32_plan(gemm_f16f32_plan_t *out,
                      int64_t M, int64_t N, int64_t K,
                      int layout_a, int layout_b, int out_type,
                      int64_t lda, int64_t ldb, int64_t ldc,
                      int64_t batch, int64_t stride_a, int64_t stride_b,
                      int64_t stride_c);

/*
 * Runs a bfloat16 plan on `stream`, asynchronously, as gemm_f16f32_run does:
 *   A, B   device pointers to bfloat16 storage (const), described by the plan.
 *   C      device pointer to bfloat16 or fp32 storage, read (beta != 0) and
 *          written.
 *   alpha, beta  fp32 scalars, by value.
 *   workspace, workspace_bytes  as gemm_f16f32_run (sized by
 *          gemm_f16f32_workspace_size on this plan).
 *   stream a hipStream_t; NULL means the default stream.
 * Rules and status codes as gemm_f16f32_run; a plan made by
 * gemm_f16f32_plan -> INVALID_ARG (nothing is launched).
 */
int gemm_bf16f32_run(gemm_f16f32_plan_t plan,
                     const void *A, const void *B, void *C,
                     float alpha, float beta,
                     void *workspace, int64_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_BF16F32_H */
