/*
 * gemm_f16f32.h -- C ABI of the MI355X (gfx950) mixed-precision GEMM.
 *
 *   C = alpha * A * B + beta * C
 *
 * A and B hold IEEE binary16 values; products are accumulated in fp32; C
 * (read when beta != 0, then written) is binary16 or fp32.  Any M, N, K from
 * 1 to several thousand; A and B each row- or column-major; strided batches.
 *
 * Pages this interface follows (titles as printed on them):
 *   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM
 *             kernel): §1.3 fixes the problem -- fp16 inputs and output, fp32
 *             accumulation, arbitrary M, N, K from 1 to thousands; §3.4 fixes
 *             the edge rule -- out-of-range elements of partial tiles,
 *             including the K remainder, contribute zero.
 *   [CATLASS] CATLASS template library page: §2.1 gives C = A * B + C as the
 *             operation; §1.1 and §1.3 make the row/column-major layout of
 *             each operand a parameter, row-major (m, n) at m * ld + n.
 *   [OPS]     CUDA operator practice page (Softmax and GEMM): §3.2 writes C
 *             row-major; §5.2 warns that 32-bit index products overflow, so
 *             every extent and offset here is 64-bit.
 * alpha and beta are the BLAS-style generalisation of [CATLASS] §2.1.
 *
 * Semantics (all indices 0-based, all extents and strides in ELEMENTS):
 *   A(b,i,k) = A[b*stride_a + i*lda + k]  (GEMM_ROW_MAJOR, lda >= K)
 *            = A[b*stride_a + i + k*lda]  (GEMM_COL_MAJOR, lda >= M)
 *   B(b,k,j) = B[b*stride_b + k*ldb + j]  (GEMM_ROW_MAJOR, ldb >= N)
 *            = B[b*stride_b + k + j*ldb]  (GEMM_COL_MAJOR, ldb >= K)
 *   C(b,i,j) = C[b*stride_c + i*ldc + j]  (always row-major, ldc >= N)
 *   C(b,i,j) <- fp32(alpha) * sum_k A(b,i,k) B(b,k,j) + fp32(beta) * C(b,i,j)
 * (with a fused epilogue, gemm_f16f32_set_epilogue: act(... + bias[j])).
 * The sum is taken in fp32 in an order the kernel chooses; the fp32 result is
 * rounded once to binary16 (round to nearest even, overflow to +-inf) for a
 * binary16 C, or stored as is for an fp32 C.  When beta == 0, C is not read
 * (NaN or garbage in C does not propagate).  Elements of A, B or C lying in
 * the padding of a leading dimension are never read and never written.
 * A column-major C is obtained by the caller by swapping operands
 * (C^T = B^T A^T).
 *
 * Ownership: the caller owns A, B, C, the stream and the workspace.  A plan
 * is host memory only: planning, running and destroying it allocate no device
 * memory, and no entry point synchronises the device or a stream.  A plan is
 * immutable once made (except through gemm_f16f32_set_epilogue), so one plan
 * may be run concurrently on several streams, each run with its own workspace.
 *
 * Workspace: some plans need device scratch memory, supplied by the caller to
 * every run (gemm_f16f32_workspace_size gives the bytes; 0 means none):
 *   - split-K (kernel name contains "_sk<slices>"): one word per output tile,
 *     counting the K slices that have finished it, in the first 4096 bytes,
 *     then slices x tiles fp32 partial tiles (64 KiB each on the 128 x 128
 *     tile, one 32 x 64, 16 x 48 ... block each on the streaming kernels);
 *   - repacking (kernel name ends in "_pka", "_pkb" or "_pkab"): dense copies
 *     of the operands whose rows do not allow 128-bit loads, rows padded to a
 *     multiple of 8 elements.
 * The workspace is 256-byte aligned and belongs to one run at a time: runs
 * that may execute at the same time (on different streams) need distinct
 * workspaces.  The counter words (bytes 0..4095) must be zero when a split-K
 * run starts; every split-K run leaves them zero when it ends.  A buffer
 * zero-filled once (gemm_f16f32_workspace_init, hipMemset, a zeroed tensor)
 * therefore serves any sequence of runs of any plans.
 * gemm_f16f32_run is asynchronous on the given stream: A, B, C and the
 * workspace must stay valid until the stream has passed the launched kernels.
 * A plan may be destroyed as soon as gemm_f16f32_run returns.
 *
 * Errors: every function returns a status code (GEMM_OK == 0 or a negative
 * GEMM_ERR_*); no exception crosses this boundary and there is no global
 * error state.  Faults raised by the device while the kernel runs are
 * reported by the HIP runtime at the caller's next synchronisation.
 */
#ifndef GEMM_F16F32_H
#define GEMM_F16F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemm_f16f32_plan_s *gemm_f16f32_plan_t; /* opaque, host only */

enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 };  /* storage of A and of B */
enum { GEMM_OUT_F16 = 0, GEMM_OUT_F32 = 1 };      /* element type of C     */

/* Activation of the fused epilogue (gemm_f16f32_set_epilogue). */
enum { GEMM_ACT_NONE = 0, GEMM_ACT_RELU = 1, GEMM_ACT_GELU = 2, GEMM_ACT_SILU = 3 };

enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = -1,  /* argument violates a rule stated below    */
    GEMM_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels cover */
    GEMM_ERR_HIP = -3,          /* the HIP runtime refused the launch       */
    GEMM_ERR_NOMEM = -4,        /* host allocation of a plan failed         */
    GEMM_ERR_SCRATCH = -5       /* gemm_f16f32_run_noalloc: the plan needs
                                   more scratch than the library holds      */
};

/*
 * Validates a problem description and chooses the kernel for it.  No device
 * work and no HIP call is made; the call can be made on a machine without a
 * GPU.
 *   out                 receives the new plan (set to NULL on failure).
 *   M, N, K             extents; negative -> INVALID_ARG.  M == 0 or N == 0
 *                       makes a plan whose run is a no-op; K == 0 makes
 *                       C <- beta * C.
 *   layout_a, layout_b  GEMM_ROW_MAJOR or GEMM_COL_MAJOR, else INVALID_ARG.
 *   out_type            GEMM_OUT_F16 or GEMM_OUT_F32, else INVALID_ARG.
 *   lda, ldb, ldc       leading dimensions, >= the minimum given in the
 *                       header comment and >= 1, else INVALID_ARG.
 *   batch               >= 1, else INVALID_ARG.
 *   stride_a/b/c        element distance between consecutive batch items;
 *                       ignored when batch == 1; must be >= 0, and
 *                       stride_c must be at least M*ldc (batch items of C may
 *                       not overlap), else INVALID_ARG.
 * Leading dimensions of any size are accepted.  The kernels address an
 * operand tile with 32-bit byte offsets, so an A or B whose leading dimension
 * exceeds 2^22 elements is copied into the workspace (both operands are then
 * repacked) before the product; an operand row or column that is itself
 * longer than 2^22 elements (lda > 2^22 would then be unavoidable) ->
 * UNSUPPORTED.
 */
int gemm_f16f32_plan(gemm_f16f32_plan_t *out,
                     int64_t M, int64_t N, int64_t K,
                     int layout_a, int layout_b, int out_type,
                     int64_t lda, int64_t ldb, int64_t ldc,
                     int64_t batch, int64_t stride_a, int64_t stride_b,
                     int64_t stride_c);

/*
 * Device workspace, in bytes, that gemm_f16f32_run needs for this plan
 * (0: none; the plan runs with workspace == NULL).
 *   flags  0: operands at 16-byte-aligned addresses (torch allocations are).
 *          GEMM_WS_ANY_ALIGNMENT: enough to also repack operands whose
 *          pointers turn out not to be 16-byte aligned at run time (a run
 *          given less reads such operands in place with element-wide loads:
 *          correct, slower).
 *   bytes  receives the size.
 * Host only, no HIP call.  NULL plan or bytes, unknown flags -> INVALID_ARG.
 */
enum { GEMM_WS_ANY_ALIGNMENT = 1 };
int gemm_f16f32_workspace_size(gemm_f16f32_plan_t plan, int flags, int64_t *bytes);

/*
 * Prepares a workspace for its first run: zero-fills its counter words
 * (the first min(bytes, 4096) bytes) with one small kernel launched on
 * `stream`, asynchronously.  Nothing is allocated.  Needed once per buffer
 * (runs leave the counters zero); a buffer already zero-filled needs no call.
 *   workspace  device pointer (256-byte aligned), or NULL when bytes == 0.
 * NULL with bytes > 0, bytes < 0 or a misaligned pointer -> INVALID_ARG;
 * a failed launch -> GEMM_ERR_HIP.
 */
int gemm_f16f32_workspace_init(void *workspace, int64_t bytes, void *stream);

/*
 * Runs a plan: launches its kernels on `stream` (the GEMM, preceded by one
 * copy kernel when operands are repacked) and returns without waiting.  No
 * device memory is allocated and nothing is synchronised.
 *   A, B   device pointers to binary16 storage (const), described by the plan.
 *   C      device pointer to binary16 or fp32 storage, read (beta != 0) and
 *          written.
 *   alpha, beta  fp32 scalars, by value.
 *   workspace, workspace_bytes  device scratch owned by the caller (see
 *          Ownership): at least gemm_f16f32_workspace_size(plan, 0) bytes,
 *          256-byte aligned, counter words zero; NULL and 0 for a plan that
 *          needs none.
 *   stream a hipStream_t; NULL means the default stream.
 * Rules: plan != NULL; A, B, C non-NULL unless the plan's M*N == 0 (then the
 * call is a no-op and returns GEMM_OK) -- else INVALID_ARG.  The address range
 * of C must not overlap those of A, B or the workspace -> INVALID_ARG.  A
 * workspace smaller than the plan needs, misaligned or NULL with a nonzero
 * size -> INVALID_ARG.  Pointer alignment of A and B is never an error:
 * 16-byte-aligned operands whose leading dimensions, contiguous extents and
 * batch strides are multiples of 8 are read in place with 128-bit loads;
 * others are either copied first into the workspace (direct and streaming
 * kernels, when the workspace holds the copy) or read with element-wide
 * loads, with the same results up to summation order.  A failed launch ->
 * GEMM_ERR_HIP.
 */
int gemm_f16f32_run(gemm_f16f32_plan_t plan,
                    const void *A, const void *B, void *C,
                    float alpha, float beta,
                    void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gemm_f16f32_run without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is the library's own
 * static device array of 64 MiB per device, held from the library's first
 * use on a device until the process ends; on the first call on a device its
 * counter words are zero-filled by a small kernel on `stream`.  Nothing is
 * allocated or synchronised, at any call.
 *   plan   a plan of either input type (gemm_f16f32_plan or gemm_bf16f32_plan).
 *   A, B, C, alpha, beta, stream  as gemm_f16f32_run (for a bfloat16 plan,
 *          as gemm_bf16f32_run).
 * A plan whose gemm_f16f32_workspace_size(plan, 0) exceeds 64 MiB ->
 * GEMM_ERR_SCRATCH, before any HIP call.  Operands at misaligned addresses
 * are repacked into the array when the copies fit, else read in place.
 * Every call on a device shares that device's array (which keeps the last
 * call's contents): calls on one device that may execute at the same time --
 * on different streams, or from different threads -- race on it and must be
 * serialised by the caller.  Other rules and status codes as gemm_f16f32_run.
 */
int gemm_f16f32_run_noalloc(gemm_f16f32_plan_t plan,
                            const void *A, const void *B, void *C,
                            float alpha, float beta, void *stream);

/*
 * Sets the plan's fused epilogue, used by every later run of the plan:
 *   C(b,i,j) <- act( fp32(alpha) * sum_k A(b,i,k) B(b,k,j)
 *                    + fp32(beta) * C(b,i,j) + bias[j] )
 * in fp32, then rounded once to C's type.  This is the pages' "keep the GEMM
 * main loop, replace the epilogue" pattern ([CATLASS] §5.2) in the form a
 * linear layer needs: a per-column bias, the residual as beta * C, and one
 * of the activations
 *   GEMM_ACT_NONE  x
 *   GEMM_ACT_RELU  max(x, 0)
 *   GEMM_ACT_GELU  x * Phi(x) = x/2 * erfc(-x / sqrt(2))   (exact GELU)
 *   GEMM_ACT_SILU  x / (1 + exp(-x))
 * applied last (after the residual add).
 *   plan        a plan of either input type (gemm_f16f32_plan or
 *               gemm_bf16f32_plan).
 *   bias        device pointer to N fp32 values (one per column of C, shared
 *               by all rows and batch items; 4-byte aligned), or NULL for no
 *               bias.  Owned by the caller; read by the runs, so it must stay
 *               valid until the stream has passed them, and must not overlap
 *               C (checked at run -> INVALID_ARG).
 *   activation  GEMM_ACT_*.
 * Host only, no HIP call.  NULL plan, a misaligned bias or an unknown
 * activation -> INVALID_ARG (the plan is left unchanged).  Setting NULL and
 * GEMM_ACT_NONE restores the plain GEMM.  A plan with an epilogue runs the
 * epilogue form of the same kernel; gemm_f16f32_plan_kernel reports the same
 * name.  Changing the epilogue of a plan
 * while one of its runs may still be launched from another thread is a race.
 */
int gemm_f16f32_set_epilogue(gemm_f16f32_plan_t plan, const void *bias, int activation);

/*
 * Makes the plan's later runs the linear layer fused with its residual and
 * LayerNorm ([CATLASS] opening paragraph; the page names the fusion, this is
 * its plainest form, a post-norm layer):
 *   Z(b,i,j) = fp32(alpha) * sum_k A(b,i,k) B(b,k,j) + fp32(beta) * C(b,i,j) + bias[j]
 *   C(b,i,j) <- (Z(b,i,j) - mu) / sqrt(var + eps) * gamma[j] + beta_ln[j]
 * with mu and var the mean and the biased variance (divided by N) of row
 * (b, i) of Z, all in fp32, then one rounding to C's type.  The bias is the
 * one set with gemm_f16f32_set_epilogue (or none); the activation must be
 * GEMM_ACT_NONE.
 *   plan        a plan of either input type.
 *   gamma, beta_ln  device pointers to N fp32 values each (4-byte aligned),
 *               owned by the caller and read by the runs; gamma == NULL
 *               removes the normalisation (beta_ln is then ignored).
 *   eps         >= 0 and finite.
 * Host only, no HIP call.  NULL plan, a misaligned or missing beta_ln, a bad
 * eps, or an activation set on the plan -> INVALID_ARG (plan unchanged);
 * afterwards gemm_f16f32_set_epilogue refuses an activation.
 * Such a plan needs more workspace -- gemm_f16f32_workspace_size, queried
 * after this call, includes it: Z in fp32 (batch * M * (N rounded up to 4)
 * * 4 bytes) occupies the workspace's last bytes.  A run makes two launches:
 * the GEMM writing Z, then one workgroup per row normalising it into C.
 * Changing the setting while a run of the plan may still be launched from
 * another thread is a race.
 */
int gemm_f16f32_set_layernorm(gemm_f16f32_plan_t plan, const void *gamma, const void *beta_ln,
                              float eps);

/* Frees a plan (host memory only; runs already launched are unaffected).
 * NULL is a no-op.  Returns GEMM_OK. */
int gemm_f16f32_destroy(gemm_f16f32_plan_t plan);

/* A static, NUL-terminated description of a status code (never NULL). */
const char *gemm_f16f32_status_string(int status);

/*
 * Name of the kernel configuration the plan chose, as a NUL-terminated
 * string owned by the plan (valid until it is destroyed), or "none" for a
 * no-op plan and "invalid" for NULL.  Diagnostic only.  Form:
 * gemm_<tile>_<nn|nt|tn|tt>_<path>[_sk<slices>][_pka|_pkb|_pkab], where path
 * is "direct" (direct or streaming kernel), "vec16" (staged tile, 128-bit
 * loads) or "narrow" (staged tile, element-wide loads), _sk gives the K
 * slices of a split-K plan and _pk the operands repacked because of their
 * shape.
 */
const char *gemm_f16f32_plan_kernel(gemm_f16f32_plan_t plan);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16F32_H */
