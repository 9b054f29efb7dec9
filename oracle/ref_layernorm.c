/*
 * CPU oracle for the linear layer fused with its residual and LayerNorm:
 *   Z = alpha * A B + beta * C + bias[n]
 *   Y[i, n] = (Z[i, n] - mu_i) / sqrt(var_i + eps) * gamma[n] + beta_ln[n]
 *   mu_i = (1/N) sum_n Z[i, n],  var_i = (1/N) sum_n (Z[i, n] - mu_i)^2
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or shares any code, header or table with it.
 *
 * Pages cited (titles as printed on them):
 *   [CATLASS] CATLASS template library
 *             (printed title "企业官网建设流程全解析", hotelren.com/news/4584228):
 *             the opening paragraph's case is a linear layer fused with its
 *             residual and LayerNorm; §5.2 keeps the GEMM main loop and
 *             replaces the epilogue; §3 keeps reductions such as LayerNorm
 *             in fp32.
 *   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM
 *             kernel): §1.1 a fully connected layer is a GEMM.
 * The pages name the fusion, not its formula.  The plainest reading taken:
 * the residual is the GEMM's beta * C term and the bias is added before the
 * normalisation (post-norm: LayerNorm(x W^T + b + residual)); LayerNorm
 * normalises each row over its N columns with the biased variance (divided
 * by N), eps inside the square root, and a per-column scale gamma and shift
 * beta_ln.
 *
 * Z comes from oracle_gemm (the plain fp64 GEMM of ref_gemm.c, with its error
 * scale S); the row statistics are plain two-pass sums in double.  Besides Y
 * the oracle returns, per row, mu, s = sqrt(var + eps), the mean absolute
 * value of Z and the error bound term
 *   T[i, n] = |gamma_n| (2 D_i + |Z[i, n] - mu_i| D_i / s_i) / s_i
 * with D_i = 2e-3 max_n S[i, n], the first-order effect on Y of an error of
 * at most D_i in every element of the row of Z (the mean moves by at most
 * D_i, and s, a 1-Lipschitz function of the row, by at most D_i).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

int oracle_gemm(int64_t batch, int64_t M, int64_t N, int64_t K,
                int layout_a, int layout_b, int in_type, int out_type,
                int64_t lda, int64_t ldb, int64_t ldc,
                int64_t stride_a, int64_t stride_b, int64_t stride_c,
                const uint16_t *A, const uint16_t *B, const void *C,
                double alpha, double beta, const float *bias, int act,
                const int64_t *rows, int64_t nrows,
                double *ref, double *scale, int nthreads);

/* LayerNorm of one row z[0..n-1] into y; returns mu, s, mean |z| in out3. */
void oracle_layernorm_row(const double *z, int64_t n, const float *gamma, const float *beta_ln,
                          double eps, double *y, double *out3)
{
    double sum = 0.0, asum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        sum += z[j];
        asum += fabs(z[j]);
    }
    const double mu = n > 0 ? sum / (double)n : 0.0;
    double sq = 0.0;
    for (int64_t j = 0; j < n; ++j)
        sq += (z[j] - mu) * (z[j] - mu);
    const double var = n > 0 ? sq / (double)n : 0.0;
    const double s = sqrt(var + eps);
    for (int64_t j = 0; j < n; ++j)
        y[j] = (z[j] - mu) / s * (double)gamma[j] + (double)beta_ln[j];
    out3[0] = mu;
    out3[1] = s;
    out3[2] = n > 0 ? asum / (double)n : 0.0;
}

/*
 * The fused layer over a strided batch (arguments of oracle_gemm, plus gamma,
 * beta_ln: N floats each, and eps).  Results, dense:
 *   y     [batch][nrows][N]   Y
 *   t     [batch][nrows][N]   the bound term T above
 *   stats [batch][nrows][3]   mu, s, mean |Z|
 * Returns 0, -1 on bad arguments, -2 when memory runs out.
 */
int oracle_gemm_layernorm(int64_t batch, int64_t M, int64_t N, int64_t K,
                          int layout_a, int layout_b, int in_type, int out_type,
                          int64_t lda, int64_t ldb, int64_t ldc,
                          int64_t stride_a, int64_t stride_b, int64_t stride_c,
                          const uint16_t *A, const uint16_t *B, const void *C,
                          double alpha, double beta, const float *bias,
                          const float *gamma, const float *beta_ln, double eps,
                          const int64_t *rows, int64_t nrows,
                          double *y, double *t, double *stats, int nthreads)
{
    if (!gamma || !beta_ln || eps < 0.0)
        return -1;
    const int64_t total = batch * nrows * N;
    double *z = (double *)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    double *sc = (double *)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    if (!z || !sc) {
        free(z);
        free(sc);
        return -2;
    }
    int rc = oracle_gemm(batch, M, N, K, layout_a, layout_b, in_type, out_type, lda, ldb, ldc,
                         stride_a, stride_b, stride_c, A, B, C, alpha, beta, bias, 0, rows,
                         nrows, z, sc, nthreads);
    if (rc == 0) {
        for (int64_t r = 0; r < batch * nrows; ++r) {
            const double *zr = z + r * N, *sr = sc + r * N;
            double *st = stats + r * 3;
            oracle_layernorm_row(zr, N, gamma, beta_ln, eps, y + r * N, st);
            double smax = 0.0;
            for (int64_t j = 0; j < N; ++j)
                if (sr[j] > smax) smax = sr[j];
            const double Di = 2e-3 * smax, s = st[1];
            for (int64_t j = 0; j < N; ++j)
                t[r * N + j] = s > 0.0 ? fabs((double)gamma[j]) *
                                             (2.0 * Di + fabs(zr[j] - st[0]) * Di / s) / s
                                       : INFINITY;
        }
    }
    free(z);
    free(sc);
    return rc;
}
