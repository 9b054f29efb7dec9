/*
 * CPU oracle for C = alpha * A * B + beta * C with binary16 or bfloat16 A
 * and B.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or shares any code, header or table with it.
 *
 * Pages cited (titles as printed on them):
 *   [OPS]     CUDA operator practice, Softmax and GEMM
 *             (printed title "企业官网建设流程全解析", hotelren.com/news/5702447)
 *   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践"
 *             (hand-written GEMM kernel, bjdmk.com.cn/news/6079288)
 *   [CATLASS] CATLASS template library
 *             (printed title "企业官网建设流程全解析", hotelren.com/news/4584228)
 *
 * What it computes.  The tiled method reaches the plain matrix product up to
 * the order of its fp32 additions, so the oracle is that plain definition
 * written out in double precision:
 *   - [OPS] §1.3 and §4.1: a plain CPU implementation is the yardstick every
 *     kernel is compared against;
 *   - [OPS] §3.1: output (i,j) is the dot product of row i of A with column
 *     j of B, summed over k;
 *   - [CATLASS] §2.1: the GEMM is C = A*B + C; alpha and beta scale the two
 *     terms (C is not read when beta == 0, the BLAS convention);
 *   - [GEMM] §1.3: fp16 inputs, fp32 accumulation, fp16 output;
 *   - [GEMM] §6 and [CATLASS] §3.2: bfloat16 is the other 16-bit input
 *     format (the one the pages recommend for training); the same product
 *     with bfloat16 A and B and a bfloat16 or fp32 C;
 *   - [CATLASS] §5.2 (keep the GEMM main loop, replace the epilogue) and the
 *     page's opening case (a linear layer fused with its residual): an
 *     optional fused epilogue, taken here in its plainest general form
 *       C = act(alpha * A*B + beta * C + bias[n])
 *     with bias a per-column vector (residual = the beta * C term) and act
 *     one of ReLU max(x, 0), GELU x * Phi(x) = x/2 erfc(-x / sqrt 2),
 *     SiLU x / (1 + e^-x).  The scale S then includes |bias[n]| and is the
 *     scale of the pre-activation value.
 * Every product of two inputs is exact in double (11 x 11 significant bits
 * for binary16, 8 x 8 for bfloat16), and k is summed in ascending order with
 * no reassociation (-fno-fast-math).
 * Besides the value, the oracle returns the error scale
 *   S = |alpha| * sum_k |a_ik * b_kj| + |beta| * |c_ij|
 * used by the acceptance bound.
 *
 * binary16 ([GEMM] §6.1, [CATLASS] §3.2: 1 sign bit, 5 exponent bits,
 * 10 fraction bits, largest finite 65504, subnormals down to 2^-24) is
 * decoded and encoded here from the IEEE-754 definition.  bfloat16
 * ([CATLASS] §3.2: 1 sign bit, 8 exponent bits -- the exponent range of
 * fp32 -- and 7 fraction bits) is decoded and encoded from that layout with
 * the same rules: bias 127, subnormals at exponent field 0, infinities and
 * NaNs at 255.
 *
 * Parity pins live in tests/test_oracle.py: exhaustive decode against
 * numpy.float16, encode against numpy's round-to-nearest-even, exact
 * rational brute force over tiny shapes and all four layouts, closed forms
 * (all-ones, identity, K = 1) and integer-exact inputs; for bfloat16,
 * exhaustive decode against the upper half of binary32, encode against
 * torch's round-to-nearest-even, the format's landmarks and the same brute
 * force; for the epilogue, the activations against scipy (ndtr, expit), their
 * odd-part identities, Phi(1) and sigma(1), and exact brute force with a bias.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ROW_MAJOR 0
#define ORACLE_COL_MAJOR 1
#define ORACLE_OUT_F16 0
#define ORACLE_OUT_F32 1
#define ORACLE_OUT_BF16 2
#define ORACLE_IN_F16 0
#define ORACLE_IN_BF16 1
#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_GELU 2
#define ORACLE_ACT_SILU 3

/* binary16 -> double.  e = 0: f * 2^-24 (zero or subnormal);
 * 1 <= e <= 30: (1024 + f) * 2^(e - 25); e = 31: inf (f = 0) or NaN. */
double oracle_dec16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25);
    return sign ? -mag : mag;
}

/* double -> binary16, round to nearest, ties to even.  Magnitudes at or
 * above 65520 (halfway between 65504 and 2^16, a tie that goes to the even
 * neighbour 2^16) become infinity.  NaN maps to the quiet NaN 0x7E00 with
 * the input's sign. */
uint16_t oracle_enc16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00);
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7C00);
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2 with m in [0.5, 1) */
    int E = e2 - 1;         /* floor(log2(a)) */
    if (E < -14)
        E = -14;            /* subnormal range shares the 2^-24 quantum */
    double n = ldexp(a, 10 - E);     /* a / quantum, exact */
    double r = nearbyint(n);         /* default mode: nearest, ties even */
    uint32_t ri = (uint32_t)r;
    if (E == -14 && ri < 1024)
        return (uint16_t)(sign | ri); /* subnormal or zero */
    if (ri == 2048) {                  /* rounding carried into next binade */
        ri = 1024;
        E += 1;
    }
    return (uint16_t)(sign | ((uint32_t)(E + 15) << 10) | (ri - 1024));
}

/* bfloat16 -> double.  e = 0: f * 2^-133 (zero or subnormal: f 2^-7 times
 * the smallest normal 2^-126); 1 <= e <= 254: (128 + f) * 2^(e - 134);
 * e = 255: inf (f = 0) or NaN. */
double oracle_decbf16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 255;
    int f = h & 127;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -133);
    else if (e == 255)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(128 + f), e - 134);
    return sign ? -mag : mag;
}

/* double -> bfloat16, round to nearest, ties to even.  The quantum of the
 * binade [2^E, 2^(E+1)) is 2^(E-7), and 2^-133 below 2^-126.  A value that
 * rounds to 2^128 or more (from (2 - 2^-8) 2^127 up, the tie going to the
 * even neighbour 2^128) becomes infinity.  NaN maps to the quiet NaN 0x7FC0
 * with the input's sign. */
uint16_t oracle_encbf16(double x)
{
    uint16_t sgn = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sgn | 0x7FC0);
    double mag = fabs(x);
    if (mag == 0.0)
        return sgn;
    if (isinf(mag))
        return (uint16_t)(sgn | 0x7F80);
    int ex;
    frexp(mag, &ex);        /* mag = m * 2^ex with m in [0.5, 1) */
    int E = ex - 1;
    if (E > 127)
        return (uint16_t)(sgn | 0x7F80);
    if (E < -126)
        E = -126;
    double t = ldexp(mag, 7 - E);    /* mag / quantum, exact */
    double q = nearbyint(t);
    uint32_t qi = (uint32_t)q;
    if (E == -126 && qi < 128)
        return (uint16_t)(sgn | qi);   /* subnormal, or zero */
    if (qi == 256) {                   /* carried into the next binade */
        qi = 128;
        E += 1;
        if (E > 127)
            return (uint16_t)(sgn | 0x7F80);
    }
    return (uint16_t)(sgn | ((uint32_t)(E + 127) << 7) | (qi - 128));
}

/* The epilogue's activation of a pre-activation value x, by definition. */
double oracle_activate(int act, double x)
{
    switch (act) {
    case ORACLE_ACT_RELU:
        return x > 0.0 ? x : 0.0;
    case ORACLE_ACT_GELU:   /* Phi(x) = erfc(-x / sqrt 2) / 2, accurate in the left tail too */
        return 0.5 * x * erfc(-x / sqrt(2.0));
    case ORACLE_ACT_SILU:
        return x / (1.0 + exp(-x));
    default:
        return x;
    }
}

typedef struct {
    int64_t batch, M, N, K;
    int layout_a, layout_b, in_type, out_type;
    int64_t lda, ldb, ldc, stride_a, stride_b, stride_c;
    const uint16_t *A, *B;
    const void *C;
    double alpha, beta;
    const float *bias;       /* per-column bias (N values) or NULL */
    int act;                 /* ORACLE_ACT_* */
    const int64_t *rows;
    int64_t nrows;
    double *ref, *scale;
    const double *shared_bt; /* B of batch item 0 decoded once, when batch == 1 */
    int64_t lo, hi;          /* range of (b, r) work items for this thread */
    int err;
} job_t;

static double elem_a(const job_t *j, int64_t b, int64_t i, int64_t k)
{
    const uint16_t *A = j->A + b * j->stride_a;
    uint16_t h = (j->layout_a == ORACLE_ROW_MAJOR) ? A[i * j->lda + k]
                                                   : A[i + k * j->lda];
    return j->in_type == ORACLE_IN_BF16 ? oracle_decbf16(h) : oracle_dec16(h);
}

static double elem_b(const job_t *j, int64_t b, int64_t k, int64_t n)
{
    const uint16_t *B = j->B + b * j->stride_b;
    uint16_t h = (j->layout_b == ORACLE_ROW_MAJOR) ? B[k * j->ldb + n]
                                                   : B[k + n * j->ldb];
    return j->in_type == ORACLE_IN_BF16 ? oracle_decbf16(h) : oracle_dec16(h);
}

static double elem_c(const job_t *j, int64_t b, int64_t i, int64_t n)
{
    int64_t off = b * j->stride_c + i * j->ldc + n;
    if (j->out_type == ORACLE_OUT_F16)
        return oracle_dec16(((const uint16_t *)j->C)[off]);
    if (j->out_type == ORACLE_OUT_BF16)
        return oracle_decbf16(((const uint16_t *)j->C)[off]);
    return (double)((const float *)j->C)[off];
}

static void *run_job(void *arg)
{
    job_t *j = (job_t *)arg;
    const int64_t K = j->K, N = j->N;
    /* Decoded operands: one row of A (length K) and B transposed (N x K) so
     * the k loop reads both contiguously.  Only the storage changes; the
     * arithmetic below is the plain sum in ascending k. */
    double *arow = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    double *bt = NULL;
    if (!j->shared_bt)
        bt = (double *)malloc((size_t)((N * K) > 0 ? N * K : 1) * sizeof(double));
    if (!arow || (!j->shared_bt && !bt)) {
        free(arow);
        free(bt);
        j->err = 1;
        return NULL;
    }
    int64_t cur_b = -1;
    for (int64_t w = j->lo; w < j->hi; ++w) {
        int64_t b = w / j->nrows;
        int64_t r = w % j->nrows;
        int64_t i = j->rows ? j->rows[r] : r;
        if (b != cur_b && !j->shared_bt) {
            for (int64_t n = 0; n < N; ++n)
                for (int64_t k = 0; k < K; ++k)
                    bt[n * K + k] = elem_b(j, b, k, n);
            cur_b = b;
        }
        for (int64_t k = 0; k < K; ++k)
            arow[k] = elem_a(j, b, i, k);
        double *out = j->ref + (b * j->nrows + r) * N;
        double *sc = j->scale + (b * j->nrows + r) * N;
        for (int64_t n = 0; n < N; ++n) {
            const double *bc = (j->shared_bt ? j->shared_bt : bt) + n * K;
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = arow[k] * bc[k];
                s += p;
                t += fabs(p);
            }
            double cin = (j->beta != 0.0) ? elem_c(j, b, i, n) : 0.0;
            out[n] = j->alpha * s + j->beta * cin;
            sc[n] = fabs(j->alpha) * t + fabs(j->beta) * fabs(cin);
            if (j->bias) {
                out[n] += (double)j->bias[n];
                sc[n] += fabs((double)j->bias[n]);
            }
            out[n] = oracle_activate(j->act, out[n]);
        }
    }
    free(arow);
    free(bt);
    return NULL;
}

/*
 * Reference GEMM over a strided batch.
 *   A(b,i,k) = A[b*stride_a + i*lda + k] (row-major) or A[b*stride_a + i + k*lda]
 *   B(b,k,n) = B[b*stride_b + k*ldb + n] (row-major) or B[b*stride_b + k + n*ldb]
 *   C(b,i,n) = C[b*stride_c + i*ldc + n] (always row-major; binary16 bits when
 *              out_type == ORACLE_OUT_F16, float when ORACLE_OUT_F32,
 *              bfloat16 bits when ORACLE_OUT_BF16)
 * in_type: ORACLE_IN_F16 (A and B hold binary16 bits) or ORACLE_IN_BF16
 * (bfloat16 bits).
 * bias: NULL or N floats added to every row before the activation; act:
 * ORACLE_ACT_* applied last (ref holds act(x), scale the scale of x).
 * rows: optional list of nrows row indices to evaluate (NULL = all M rows,
 * nrows must then equal M).  Results: ref and scale, each batch x nrows x N,
 * dense.  alpha, beta: the fp32 scalars the caller passes, widened.
 * Returns 0, or -1 on bad arguments, -2 when memory runs out.
 */
int oracle_gemm(int64_t batch, int64_t M, int64_t N, int64_t K,
                int layout_a, int layout_b, int in_type, int out_type,
                int64_t lda, int64_t ldb, int64_t ldc,
                int64_t stride_a, int64_t stride_b, int64_t stride_c,
                const uint16_t *A, const uint16_t *B, const void *C,
                double alpha, double beta, const float *bias, int act,
                const int64_t *rows, int64_t nrows,
                double *ref, double *scale, int nthreads)
{
    if (batch < 0 || M < 0 || N < 0 || K < 0 || nrows < 0)
        return -1;
    if (in_type != ORACLE_IN_F16 && in_type != ORACLE_IN_BF16)
        return -1;
    if (out_type != ORACLE_OUT_F16 && out_type != ORACLE_OUT_F32 && out_type != ORACLE_OUT_BF16)
        return -1;
    if (act < ORACLE_ACT_NONE || act > ORACLE_ACT_SILU)
        return -1;
    if (!rows && nrows != M)
        return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M)
                return -1;
    int64_t work = batch * nrows;
    if (work == 0 || N == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > work)
        nthreads = (int)work;
    job_t *jobs = (job_t *)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    double *bt = NULL;
    if (jobs && batch == 1 && nthreads > 1)
        bt = (double *)malloc((size_t)((N * K) > 0 ? N * K : 1) * sizeof(double));
    if (!jobs || !tid || (batch == 1 && nthreads > 1 && !bt)) {
        free(jobs);
        free(tid);
        free(bt);
        return -2;
    }
    if (bt) {
        job_t probe;
        memset(&probe, 0, sizeof probe);
        probe.layout_b = layout_b; probe.ldb = ldb; probe.B = B; probe.in_type = in_type;
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < K; ++k)
                bt[n * K + k] = elem_b(&probe, 0, k, n);
    }
    for (int t = 0; t < nthreads; ++t) {
        job_t *j = &jobs[t];
        j->batch = batch; j->M = M; j->N = N; j->K = K;
        j->layout_a = layout_a; j->layout_b = layout_b; j->in_type = in_type;
        j->out_type = out_type;
        j->lda = lda; j->ldb = ldb; j->ldc = ldc;
        j->stride_a = stride_a; j->stride_b = stride_b; j->stride_c = stride_c;
        j->A = A; j->B = B; j->C = C;
        j->alpha = alpha; j->beta = beta;
        j->bias = bias; j->act = act;
        j->rows = rows; j->nrows = nrows;
        j->ref = ref; j->scale = scale;
        j->shared_bt = bt;
        j->lo = work * t / nthreads;
        j->hi = work * (t + 1) / nthreads;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0)
            break;
        started = t;
    }
    run_job(&jobs[0]);
    for (int t = started + 1; t < nthreads; ++t)   /* threads that failed to start */
        run_job(&jobs[t]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    int err = 0;
    for (int t = 0; t < nthreads; ++t)
        err |= jobs[t].err;
    free(jobs);
    free(tid);
    free(bt);
    return err ? -2 : 0;
}
