/*
 * CPU oracle for row softmax and for attention O = softmax(scale Q K^T) V.
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
 * What it computes.
 *   - Softmax of a row ([OPS] §2.1): the textbook three steps -- the row's
 *     maximum, the sum of exp(x - max), each exp(x - max) divided by that
 *     sum -- in double precision (oracle_softmax_row).
 *   - The online form of the same quantity ([OPS] §2.2): the row is consumed
 *     block by block, keeping the largest value seen so far m and the sum s
 *     of exp(x - m) over what has been seen; a new block with largest value
 *     m_new moves the reference to m' = max(m, m_new), rescales the old sum
 *     by exp(m - m') and adds exp(x - m') of the block's elements
 *     (oracle_softmax_row_online).  It exists to pin the two-pass form: both
 *     are exact definitions of the same numbers.
 *   - Attention ([GEMM] §1.1 and [CATLASS] §5.2: Q K^T is one matrix
 *     product, softmax over each row of the scores, then a product with V):
 *       s_ij = scale * sum_d Q[i,d] K[j,d],  P = softmax over j of s_i.,
 *       O[i,c] = sum_j P_ij V[j,c]
 *     with Q, K, V binary16 (decoded exactly) and everything else in double
 *     (oracle_attention).
 *   - Masking.  With `causal`, key j is visible to query i iff
 *     j <= i + (Sk - Sq): the last query sees every key (the alignment a
 *     decoder uses when Sq new queries follow Sk - Sq cached keys).  A row
 *     whose keys are all masked -- for the row softmax, a row of -inf --
 *     has no finite maximum: [OPS] §2.5 notes that the plain computation
 *     then divides 0 by 0 and produces NaN, and that such rows should be
 *     excluded by the caller or given a constant output.  The constant
 *     output taken here is zero: every P_ij (and so every O[i,c]) of such
 *     a row is 0.
 * Besides the value, oracle_attention returns per output the error scale
 * sum_j P_ij |V[j,c]| and per row the largest |score| bound
 * max_j scale * sum_d |Q[i,d] K[j,d]| over visible keys, which the
 * acceptance bound of the tests uses.
 *
 * Parity pins live in tests/test_oracle_attention.py: scipy.special.softmax,
 * the online form against the two-pass form, torch's scaled dot-product
 * attention in float64, closed forms (uniform scores give the mean of V,
 * one dominant score gives the textbook weighted average), shift and
 * permutation invariances, a pure-Python brute force on tiny shapes, and
 * planted mutants.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double oracle_dec16(uint16_t h);   /* binary16 decoder of ref_gemm.c */

/* Softmax of x[0..n-1] into y by the definition.  -inf elements get 0; a row
 * with no element above -inf (or n == 0) is all zeros. */
void oracle_softmax_row(const double *x, int64_t n, double *y)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (x[j] > m)
            m = x[j];
    if (m == -INFINITY) {
        for (int64_t j = 0; j < n; ++j)
            y[j] = 0.0;
        return;
    }
    double s = 0.0;
    for (int64_t j = 0; j < n; ++j)
        s += exp(x[j] - m);
    for (int64_t j = 0; j < n; ++j)
        y[j] = exp(x[j] - m) / s;
}

/* The same softmax through the online recurrence, `block` elements at a time. */
void oracle_softmax_row_online(const double *x, int64_t n, int64_t block, double *y)
{
    if (block < 1)
        block = 1;
    double m = -INFINITY, s = 0.0;
    for (int64_t j0 = 0; j0 < n; j0 += block) {
        int64_t j1 = j0 + block < n ? j0 + block : n;
        double m_new = -INFINITY;
        for (int64_t j = j0; j < j1; ++j)
            if (x[j] > m_new)
                m_new = x[j];
        double m2 = m > m_new ? m : m_new;
        if (m2 == -INFINITY)
            continue;                       /* nothing visible yet */
        double acc = 0.0;
        for (int64_t j = j0; j < j1; ++j)
            acc += exp(x[j] - m2);
        s = (m == -INFINITY ? 0.0 : s * exp(m - m2)) + acc;
        m = m2;
    }
    for (int64_t j = 0; j < n; ++j)
        y[j] = (m == -INFINITY) ? 0.0 : exp(x[j] - m) / s;
}

/* Row softmax of a rows x cols matrix of binary16 (in_f32 == 0) or float
 * (in_f32 != 0) values with leading dimension ld; y is rows x cols, dense. */
int oracle_softmax(int64_t rows, int64_t cols, const void *x, int in_f32, int64_t ld,
                   double *y)
{
    if (rows < 0 || cols < 0 || ld < cols)
        return -1;
    double *row = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!row)
        return -2;
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < cols; ++j)
            row[j] = in_f32 ? (double)((const float *)x)[i * ld + j]
                            : oracle_dec16(((const uint16_t *)x)[i * ld + j]);
        oracle_softmax_row(row, cols, y + i * cols);
    }
    free(row);
    return 0;
}

typedef struct {
    int64_t heads, Sq, Sk, D, Dv;
    const uint16_t *Q, *K, *V;
    int64_t q_sb, q_sh, q_ld, k_sb, k_sh, k_ld, v_sb, v_sh, v_ld;
    double scale;
    int causal;
    const int64_t *rows;
    int64_t nrows;
    double *out, *err, *smax;
    int64_t lo, hi;       /* work items (batch * heads * nrows) of this thread */
    int fail;
} attn_job_t;

static void *attn_run(void *arg)
{
    attn_job_t *j = (attn_job_t *)arg;
    const int64_t Sk = j->Sk, D = j->D, Dv = j->Dv;
    double *q = (double *)malloc((size_t)(D > 0 ? D : 1) * sizeof(double));
    double *s = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
    double *p = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
    double *a = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
    if (!q || !s || !p || !a) {
        free(q); free(s); free(p); free(a);
        j->fail = 1;
        return NULL;
    }
    for (int64_t w = j->lo; w < j->hi; ++w) {
        const int64_t bh = w / j->nrows, r = w % j->nrows;
        const int64_t b = bh / j->heads, h = bh % j->heads;
        const int64_t i = j->rows ? j->rows[r] : r;
        const uint16_t *Qb = j->Q + b * j->q_sb + h * j->q_sh;
        const uint16_t *Kb = j->K + b * j->k_sb + h * j->k_sh;
        const uint16_t *Vb = j->V + b * j->v_sb + h * j->v_sh;
        /* visible keys: all, or j <= i + Sk - Sq */
        int64_t nvis = Sk;
        if (j->causal) {
            nvis = i + Sk - j->Sq + 1;
            if (nvis < 0) nvis = 0;
            if (nvis > Sk) nvis = Sk;
        }
        for (int64_t d = 0; d < D; ++d)
            q[d] = oracle_dec16(Qb[i * j->q_ld + d]);
        double amax = 0.0;
        for (int64_t k = 0; k < Sk; ++k) {
            if (k >= nvis) {
                s[k] = -INFINITY;
                continue;
            }
            double dot = 0.0, adot = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                double prod = q[d] * oracle_dec16(Kb[k * j->k_ld + d]);
                dot += prod;
                adot += fabs(prod);
            }
            s[k] = j->scale * dot;
            a[k] = fabs(j->scale) * adot;
            if (a[k] > amax) amax = a[k];
        }
        oracle_softmax_row(s, Sk, p);
        double *o = j->out + w * Dv;
        double *e = j->err + w * Dv;
        for (int64_t c = 0; c < Dv; ++c) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < nvis; ++k) {
                double v = oracle_dec16(Vb[k * j->v_ld + c]);
                acc += p[k] * v;
                aacc += p[k] * fabs(v);
            }
            o[c] = acc;
            e[c] = aacc;
        }
        j->smax[w] = amax;
    }
    free(q); free(s); free(p); free(a);
    return NULL;
}

/*
 * Reference attention over batch x heads independent problems.
 *   Q(b,h,i,d) = Q[b*q_sb + h*q_sh + i*q_ld + d]   (binary16 bits, i < Sq, d < D)
 *   K(b,h,j,d) = K[b*k_sb + h*k_sh + j*k_ld + d]   (j < Sk)
 *   V(b,h,j,c) = V[b*v_sb + h*v_sh + j*v_ld + c]   (c < Dv)
 * scale: the factor on the scores (the caller's fp32 value, widened);
 * causal: nonzero masks key j from query i when j > i + Sk - Sq.
 * rows: optional list of nrows query rows to evaluate (NULL = all Sq rows,
 * nrows must then equal Sq).  Results, dense over (b, h, row):
 *   out  [batch][heads][nrows][Dv]  O
 *   err  [batch][heads][nrows][Dv]  sum_j P_ij |V[j,c]|
 *   smax [batch][heads][nrows]      max over visible j of scale sum_d |Q K|
 * Returns 0, -1 on bad arguments, -2 when memory runs out.
 */
int oracle_attention(int64_t batch, int64_t heads, int64_t Sq, int64_t Sk, int64_t D,
                     int64_t Dv, const uint16_t *Q, int64_t q_sb, int64_t q_sh, int64_t q_ld,
                     const uint16_t *K, int64_t k_sb, int64_t k_sh, int64_t k_ld,
                     const uint16_t *V, int64_t v_sb, int64_t v_sh, int64_t v_ld,
                     double scale, int causal, const int64_t *rows, int64_t nrows,
                     double *out, double *err, double *smax, int nthreads)
{
    if (batch < 0 || heads < 0 || Sq < 0 || Sk < 0 || D < 0 || Dv < 0 || nrows < 0)
        return -1;
    if (!rows && nrows != Sq)
        return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= Sq)
                return -1;
    const int64_t work = batch * heads * nrows;
    if (work == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > work)
        nthreads = (int)work;
    attn_job_t *jobs = (attn_job_t *)calloc((size_t)nthreads, sizeof(attn_job_t));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -2;
    }
    for (int t = 0; t < nthreads; ++t) {
        attn_job_t *j = &jobs[t];
        j->heads = heads; j->Sq = Sq; j->Sk = Sk; j->D = D; j->Dv = Dv;
        j->Q = Q; j->K = K; j->V = V;
        j->q_sb = q_sb; j->q_sh = q_sh; j->q_ld = q_ld;
        j->k_sb = k_sb; j->k_sh = k_sh; j->k_ld = k_ld;
        j->v_sb = v_sb; j->v_sh = v_sh; j->v_ld = v_ld;
        j->scale = scale; j->causal = causal;
        j->rows = rows; j->nrows = nrows;
        j->out = out; j->err = err; j->smax = smax;
        j->lo = work * t / nthreads;
        j->hi = work * (t + 1) / nthreads;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, attn_run, &jobs[t]) != 0)
            break;
        started = t;
    }
    attn_run(&jobs[0]);
    for (int t = started + 1; t < nthreads; ++t)
        attn_run(&jobs[t]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    int fail = 0;
    for (int t = 0; t < nthreads; ++t)
        fail |= jobs[t].fail;
    free(jobs);
    free(tid);
    return fail ? -2 : 0;
}
