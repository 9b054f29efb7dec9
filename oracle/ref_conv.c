/*
 * CPU oracle for 2-D convolution (cross-correlation, as neural networks use
 * it) of binary16 activations and filters:
 *   y[n, p, q, k] = alpha * sum_{r, s, c} x[n, p*sh - ph + r*dh, q*sw - pw + s*dw, c]
 *                                         * w[k, r, s, c]
 *                   + beta * y_old[n, p, q, k] + bias[k],   then an activation
 * with input positions outside the H x W image contributing zero.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or shares any code, header or table with it.
 *
 * Pages cited (titles as printed on them):
 *   [CATLASS] CATLASS template library
 *             (printed title "企业官网建设流程全解析", hotelren.com/news/4584228):
 *             §5.1 a convolution is a four-deep loop that becomes a matrix
 *             product by unrolling input windows (im2col) and filters; the
 *             implicit form reads the unrolled matrix on the fly, mapping row
 *             m to an input position and column n to a filter position.
 *   [GEMM]    "手写GEMM内核：矩阵乘法性能优化的完整工程实践" (hand-written GEMM
 *             kernel): §1.1 convolution via im2col is a GEMM.
 * What the oracle computes is the convolution's definition, summed directly
 * over (r, s, c) in that order in double precision (every product of two
 * binary16 values is exact), not through any unrolled matrix.  Layouts: x is
 * NHWC (channels innermost), w is KRSC, y is NPQK -- the layouts in which the
 * unrolled matrices are row-major A (M = N P Q rows of R S C) and
 * column-major B, and y is the row-major C.  Output size:
 *   P = (H + 2 ph - dh (R - 1) - 1) / sh + 1,  Q likewise with W, pw, dw, S, sw.
 * Besides y it returns the error scale
 *   S = |alpha| sum |x w| + |beta| |y_old| + |bias[k]|
 * of the acceptance bound (that of the GEMM of the same products).
 * act: 0 none, 1 ReLU (the activations of ref_gemm.c's epilogue).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

double oracle_dec16(uint16_t h);            /* binary16 decoder of ref_gemm.c */
double oracle_activate(int act, double x);  /* epilogue activations of ref_gemm.c */

/* Output extent of one spatial dimension, or -1 when the window does not fit. */
int64_t oracle_conv_out_dim(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dil)
{
    const int64_t span = dil * (k - 1) + 1;
    if (in + 2 * pad < span || stride < 1)
        return -1;
    return (in + 2 * pad - span) / stride + 1;
}

typedef struct {
    int64_t N, H, W, C, K, R, S, P, Q, sh, sw, ph, pw, dh, dw;
    const uint16_t *x, *w;
    const void *y_old;
    int out_f32;
    double alpha, beta;
    const float *bias;
    int act;
    const int64_t *rows;      /* output pixels m = (n P + p) Q + q to evaluate, or NULL */
    int64_t nrows;
    double *ref, *scale;      /* nrows x K */
    int64_t lo, hi;
} conv_job_t;

static void *conv_run(void *arg)
{
    conv_job_t *j = (conv_job_t *)arg;
    for (int64_t t = j->lo; t < j->hi; ++t) {
        const int64_t m = j->rows ? j->rows[t] : t;
        const int64_t n = m / (j->P * j->Q), pq = m % (j->P * j->Q);
        const int64_t p = pq / j->Q, q = pq % j->Q;
        for (int64_t k = 0; k < j->K; ++k) {
            double s = 0.0, a = 0.0;
            for (int64_t r = 0; r < j->R; ++r) {
                const int64_t ih = p * j->sh - j->ph + r * j->dh;
                if (ih < 0 || ih >= j->H)
                    continue;
                for (int64_t ss = 0; ss < j->S; ++ss) {
                    const int64_t iw = q * j->sw - j->pw + ss * j->dw;
                    if (iw < 0 || iw >= j->W)
                        continue;
                    const uint16_t *xp = j->x + ((n * j->H + ih) * j->W + iw) * j->C;
                    const uint16_t *wp = j->w + ((k * j->R + r) * j->S + ss) * j->C;
                    for (int64_t c = 0; c < j->C; ++c) {
                        const double prod = oracle_dec16(xp[c]) * oracle_dec16(wp[c]);
                        s += prod;
                        a += fabs(prod);
                    }
                }
            }
            double yo = 0.0;
            if (j->beta != 0.0) {
                const int64_t off = m * j->K + k;
                yo = j->out_f32 ? (double)((const float *)j->y_old)[off]
                                : oracle_dec16(((const uint16_t *)j->y_old)[off]);
            }
            double v = j->alpha * s + j->beta * yo;
            double sc = fabs(j->alpha) * a + fabs(j->beta) * fabs(yo);
            if (j->bias) {
                v += (double)j->bias[k];
                sc += fabs((double)j->bias[k]);
            }
            j->ref[t * j->K + k] = oracle_activate(j->act, v);
            j->scale[t * j->K + k] = sc;
        }
    }
    return NULL;
}

/*
 * Reference convolution.  x: N*H*W*C binary16 (NHWC), w: K*R*S*C (KRSC),
 * y_old: N*P*Q*K (NPQK, binary16 or fp32 when out_f32), read when beta != 0.
 * rows: optional list of output pixels m (NULL = all N*P*Q).  Results ref and
 * scale, nrows x K each.  Returns 0, or -1 on bad arguments.
 */
int oracle_conv2d(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                  int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                  const uint16_t *x, const uint16_t *w, const void *y_old, int out_f32,
                  double alpha, double beta, const float *bias, int act,
                  const int64_t *rows, int64_t nrows, double *ref, double *scale, int nthreads)
{
    if (N < 0 || H < 1 || W < 1 || C < 1 || K < 0 || R < 1 || S < 1 || dh < 1 || dw < 1 ||
        ph < 0 || pw < 0)
        return -1;
    const int64_t P = oracle_conv_out_dim(H, R, sh, ph, dh), Q = oracle_conv_out_dim(W, S, sw, pw, dw);
    if (P < 0 || Q < 0)
        return -1;
    const int64_t M = N * P * Q;
    if (!rows && nrows != M)
        return -1;
    if (rows)
        for (int64_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= M)
                return -1;
    if (nrows == 0 || K == 0)
        return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;
    conv_job_t *jobs = (conv_job_t *)calloc((size_t)nthreads, sizeof(conv_job_t));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -2;
    }
    for (int t = 0; t < nthreads; ++t) {
        conv_job_t *j = &jobs[t];
        j->N = N; j->H = H; j->W = W; j->C = C; j->K = K; j->R = R; j->S = S;
        j->P = P; j->Q = Q; j->sh = sh; j->sw = sw; j->ph = ph; j->pw = pw; j->dh = dh; j->dw = dw;
        j->x = x; j->w = w; j->y_old = y_old; j->out_f32 = out_f32;
        j->alpha = alpha; j->beta = beta; j->bias = bias; j->act = act;
        j->rows = rows; j->nrows = nrows; j->ref = ref; j->scale = scale;
        j->lo = nrows * t / nthreads;
        j->hi = nrows * (t + 1) / nthreads;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, conv_run, &jobs[t]) != 0)
            break;
        started = t;
    }
    conv_run(&jobs[0]);
    for (int t = started + 1; t < nthreads; ++t)
        conv_run(&jobs[t]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
    return 0;
}
