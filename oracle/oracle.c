/*
 * oracle.c -- plain, slow CPU oracle for row-wise softmax with the online
 * normalizer, computed in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library; its only contact with the GPU side is the seeded input arrays.
 *
 * Sources followed (page title, then the section on that page):
 *   [SAFE]   "OnlineSoftmax: Online normalizer calculation for softmax",
 *            section 2 "Original softmax", the safe-softmax paragraph
 *            (max, then sum of exp(x - max), then divide), and
 *            "CUDA算子优化(3)：Softmax", section "Softmax的cpu实现".
 *   [ONLINE] same paper summary, section 3.1 (the recurrence for m_j, d_j).
 *   [OPLUS]  same paper summary, section 3.3 (the binary operator on (m, d)).
 *   [IDENT]  "第 7 课：Online Softmax 与可结合状态", section 3 (the identity
 *            state (-inf, 0)).
 *   [TOPK]   same paper summary, section 4 "Softmax and top-k fusion"
 *            (probabilities of the K largest logits, relative to the whole
 *            row).  The oracle does not fuse anything: it sorts the whole row.
 *   [LSE]    "6.2 FlashAttention V2 chi tiết", sections 6.1 and 7.1 (the
 *            per-row logsumexp L = m + log(l) kept in place of m and l).
 *   [NAIVE]  the paper summary, section 2 "Original softmax", its first
 *            paragraph: y_i = e^{x_i} / sum_j e^{x_j} in two passes (the sum,
 *            then the division), no maximum subtracted.
 *   [SELECT] the paper summary, section 4, the access table: the TopK stage
 *            of the unfused pipelines reads the probabilities and keeps the K
 *            largest; here the K largest entries of any row, returned as the
 *            entries themselves (no exponential, no normaliser).
 *
 * Readings taken where the pages are silent:
 *   - An element equal to -inf contributes e^{-inf} = 0 and leaves the state
 *     unchanged; a row (or prefix) made only of -inf has the identity state
 *     (-inf, 0).  Its softmax is 0/0 = NaN.
 *   - NaN or +inf in a row makes every output of that row NaN (plain IEEE
 *     propagation through exp and the sum), d and the logsumexp included, also
 *     when every other entry is -inf; m stays the maximum of the non-NaN
 *     entries (-inf if there are none).
 *   - Top-K order is the total order (value descending, index ascending); the
 *     probability of a selected logit u is e^{u - m}/d over the whole row.
 *   - The logsumexp of a row is log(sum_j e^{x_j}), written as m + log(d)
 *     (an exact identity that keeps the sum finite): -inf for an empty or
 *     all -inf row, NaN for a row holding NaN or +inf, as for the softmax.
 *   - The naive softmax is the definition computed as printed, in double:
 *     e^x overflows to +inf past x = 709.78 and underflows to 0 below about
 *     -745, and the results then follow IEEE (inf/inf and 0/0 are NaN).  That
 *     is the failure the page describes; the oracle does not guard it.
 *   - Selection orders entries like the top-K, (value descending, index
 *     ascending); rows holding NaN have no specified order.
 *
 * Every floating-point step is IEEE double with no reassociation: build with
 * -ffp-contract=off and without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 carries the top 16 bits of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t word = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------------- */
/* [SAFE] one row: pass 1 max, pass 2 sum, pass 3 normalise.                */
/* ---------------------------------------------------------------------- */

static double row_max(const double *x, int64_t n)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (x[j] > m)
            m = x[j];
    return m;
}

static double row_sum_exp(const double *x, int64_t n, double m)
{
    if (m == -INFINITY) {
        /* No entry above -inf: the -inf entries contribute nothing (the
         * identity state), but a NaN entry still makes the sum NaN. */
        for (int64_t j = 0; j < n; ++j)
            if (x[j] != x[j])
                return NAN;
        return 0.0;
    }
    double d = 0.0;
    for (int64_t j = 0; j < n; ++j)
        d += exp(x[j] - m);
    return d;
}

static void row_softmax(const double *x, int64_t n, double *y)
{
    double m = row_max(x, n);
    double d = row_sum_exp(x, n, m);
    for (int64_t j = 0; j < n; ++j)
        y[j] = exp(x[j] - m) / d;
}

/* Widen rows [0, rows) of fp32 / bf16 input one row at a time. */
static void widen_row_f32(const float *src, int64_t n, double *dst)
{
    for (int64_t j = 0; j < n; ++j)
        dst[j] = (double)src[j];
}

static void widen_row_bf16(const uint16_t *src, int64_t n, double *dst)
{
    for (int64_t j = 0; j < n; ++j)
        dst[j] = bf16_bits_to_double(src[j]);
}

/* y[r, :] = softmax(x[r, :]) for an fp32 input, result in double.
 * Returns 0, or -1 if scratch memory could not be allocated. */
int oracle_softmax_f32(const float *x, int64_t rows, int64_t cols, double *y)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_f32(x + r * cols, cols, buf);
        row_softmax(buf, cols, y + r * cols);
    }
    free(buf);
    return 0;
}

/* Same for bf16 input given as raw 16-bit patterns. */
int oracle_softmax_bf16(const uint16_t *x, int64_t rows, int64_t cols, double *y)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_bf16(x + r * cols, cols, buf);
        row_softmax(buf, cols, y + r * cols);
    }
    free(buf);
    return 0;
}

/* Per-row normaliser state by the plain definition: m = max, d = sum e^{x-m}. */
int oracle_stats_f32(const float *x, int64_t rows, int64_t cols, double *m, double *d)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_f32(x + r * cols, cols, buf);
        m[r] = row_max(buf, cols);
        d[r] = row_sum_exp(buf, cols, m[r]);
    }
    free(buf);
    return 0;
}

int oracle_stats_bf16(const uint16_t *x, int64_t rows, int64_t cols, double *m, double *d)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_bf16(x + r * cols, cols, buf);
        m[r] = row_max(buf, cols);
        d[r] = row_sum_exp(buf, cols, m[r]);
    }
    free(buf);
    return 0;
}

/* [LSE] per-row logsumexp log(sum_j e^{x_j}) = m + log(sum_j e^{x_j - m}),
 * from the plain-definition m and d above; the empty and all -inf rows
 * (d = 0) give -inf. */
static double row_logsumexp(const double *x, int64_t n)
{
    const double m = row_max(x, n);
    const double d = row_sum_exp(x, n, m);
    return (d == 0.0) ? -INFINITY : m + log(d);
}

int oracle_logsumexp_f32(const float *x, int64_t rows, int64_t cols, double *lse)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_f32(x + r * cols, cols, buf);
        lse[r] = row_logsumexp(buf, cols);
    }
    free(buf);
    return 0;
}

int oracle_logsumexp_bf16(const uint16_t *x, int64_t rows, int64_t cols, double *lse)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_bf16(x + r * cols, cols, buf);
        lse[r] = row_logsumexp(buf, cols);
    }
    free(buf);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* [ONLINE] the recurrence, one element at a time, in the pages' order:     */
/*   m_j = max(m_{j-1}, x_j);  d_j = d_{j-1} e^{m_{j-1} - m_j} + e^{x_j - m_j} */
/* starting from the identity (m_0, d_0) = (-inf, 0).                       */
/* ---------------------------------------------------------------------- */
void oracle_online_state(const double *x, int64_t n, double *m_out, double *d_out)
{
    double m_prev = -INFINITY;
    double d_prev = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double m_new = fmax(m_prev, x[j]);
        if (m_new == -INFINITY)
            continue; /* x_j = -inf on an empty prefix: state stays the identity */
        double d_new = d_prev * exp(m_prev - m_new) + exp(x[j] - m_new);
        m_prev = m_new;
        d_prev = d_new;
    }
    *m_out = m_prev;
    *d_out = d_prev;
}

/* ---------------------------------------------------------------------- */
/* [OPLUS] (m1,d1) (+) (m2,d2) = (max, d1 e^{m1-max} + d2 e^{m2-max}),      */
/* with the identity (-inf, 0) handled exactly [IDENT].                     */
/* ---------------------------------------------------------------------- */
void oracle_combine(double m1, double d1, double m2, double d2, double *m_out, double *d_out)
{
    if (m1 == -INFINITY) {
        *m_out = m2;
        *d_out = d2;
        return;
    }
    if (m2 == -INFINITY) {
        *m_out = m1;
        *d_out = d1;
        return;
    }
    double m = fmax(m1, m2);
    *m_out = m;
    *d_out = d1 * exp(m1 - m) + d2 * exp(m2 - m);
}

/* ---------------------------------------------------------------------- */
/* [TOPK] brute force: sort the whole row under (value desc, index asc),    */
/* keep the first K, and give each its probability over the whole row.      */
/* ---------------------------------------------------------------------- */
typedef struct {
    double value;
    int64_t index;
} ranked_t;

static int rank_order(const void *pa, const void *pb)
{
    const ranked_t *a = (const ranked_t *)pa;
    const ranked_t *b = (const ranked_t *)pb;
    if (a->value > b->value)
        return -1;
    if (a->value < b->value)
        return 1;
    if (a->index < b->index)
        return -1;
    if (a->index > b->index)
        return 1;
    return 0;
}

/* One widened row: its K best entries under (value desc, index asc), with
 * probabilities e^{u - m}/d over the whole row, into probs[0..K), idx[0..K). */
static void topk_row(const double *buf, int64_t cols, int K, ranked_t *order, double *probs, int32_t *idx)
{
    double m = row_max(buf, cols);
    double d = row_sum_exp(buf, cols, m);
    for (int64_t j = 0; j < cols; ++j) {
        order[j].value = buf[j];
        order[j].index = j;
    }
    qsort(order, (size_t)cols, sizeof(ranked_t), rank_order);
    for (int k = 0; k < K; ++k) {
        probs[k] = exp(order[k].value - m) / d;
        idx[k] = (int32_t)order[k].index;
    }
}

/* probs[r*K + k], idx[r*K + k] for k = 0..K-1, best first, for an fp32 input.
 * Returns 0, -1 on allocation failure, -2 if K is out of [1, cols]. */
int oracle_topk_f32(const float *x, int64_t rows, int64_t cols, int K, double *probs, int32_t *idx)
{
    if (K < 1 || (int64_t)K > cols)
        return -2;
    double *buf = (double *)malloc((size_t)cols * sizeof(double));
    ranked_t *order = (ranked_t *)malloc((size_t)cols * sizeof(ranked_t));
    if (!buf || !order) {
        free(buf);
        free(order);
        return -1;
    }
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_f32(x + r * cols, cols, buf);
        topk_row(buf, cols, K, order, probs + r * K, idx + r * K);
    }
    free(buf);
    free(order);
    return 0;
}

/* The same for bf16 input given as raw 16-bit patterns (widened exactly). */
int oracle_topk_bf16(const uint16_t *x, int64_t rows, int64_t cols, int K, double *probs, int32_t *idx)
{
    if (K < 1 || (int64_t)K > cols)
        return -2;
    double *buf = (double *)malloc((size_t)cols * sizeof(double));
    ranked_t *order = (ranked_t *)malloc((size_t)cols * sizeof(ranked_t));
    if (!buf || !order) {
        free(buf);
        free(order);
        return -1;
    }
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_bf16(x + r * cols, cols, buf);
        topk_row(buf, cols, K, order, probs + r * K, idx + r * K);
    }
    free(buf);
    free(order);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* [NAIVE] y_i = e^{x_i} / sum_j e^{x_j}: pass 1 sums e^{x_j}, pass 2       */
/* divides; no maximum is subtracted.                                       */
/* ---------------------------------------------------------------------- */
static void row_naive_softmax(const double *x, int64_t n, double *y)
{
    double d = 0.0;
    for (int64_t j = 0; j < n; ++j)
        d += exp(x[j]);
    for (int64_t j = 0; j < n; ++j)
        y[j] = exp(x[j]) / d;
}

int oracle_naive_softmax_f32(const float *x, int64_t rows, int64_t cols, double *y)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_f32(x + r * cols, cols, buf);
        row_naive_softmax(buf, cols, y + r * cols);
    }
    free(buf);
    return 0;
}

int oracle_naive_softmax_bf16(const uint16_t *x, int64_t rows, int64_t cols, double *y)
{
    double *buf = (double *)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
    if (!buf)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_bf16(x + r * cols, cols, buf);
        row_naive_softmax(buf, cols, y + r * cols);
    }
    free(buf);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* [SELECT] brute force: sort the whole row under (value desc, index asc)   */
/* and keep the first K entries and their columns.                          */
/* ---------------------------------------------------------------------- */
static void select_row(const double *buf, int64_t cols, int K, ranked_t *order, double *vals, int32_t *idx)
{
    for (int64_t j = 0; j < cols; ++j) {
        order[j].value = buf[j];
        order[j].index = j;
    }
    qsort(order, (size_t)cols, sizeof(ranked_t), rank_order);
    for (int k = 0; k < K; ++k) {
        vals[k] = order[k].value;
        idx[k] = (int32_t)order[k].index;
    }
}

/* vals[r*K + k], idx[r*K + k] for k = 0..K-1, best first, for an fp32 input.
 * Returns 0, -1 on allocation failure, -2 if K is out of [1, cols]. */
int oracle_topk_select_f32(const float *x, int64_t rows, int64_t cols, int K, double *vals, int32_t *idx)
{
    if (K < 1 || (int64_t)K > cols)
        return -2;
    double *buf = (double *)malloc((size_t)cols * sizeof(double));
    ranked_t *order = (ranked_t *)malloc((size_t)cols * sizeof(ranked_t));
    if (!buf || !order) {
        free(buf);
        free(order);
        return -1;
    }
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_f32(x + r * cols, cols, buf);
        select_row(buf, cols, K, order, vals + r * K, idx + r * K);
    }
    free(buf);
    free(order);
    return 0;
}

/* The same for bf16 input given as raw 16-bit patterns (widened exactly). */
int oracle_topk_select_bf16(const uint16_t *x, int64_t rows, int64_t cols, int K, double *vals, int32_t *idx)
{
    if (K < 1 || (int64_t)K > cols)
        return -2;
    double *buf = (double *)malloc((size_t)cols * sizeof(double));
    ranked_t *order = (ranked_t *)malloc((size_t)cols * sizeof(ranked_t));
    if (!buf || !order) {
        free(buf);
        free(order);
        return -1;
    }
    for (int64_t r = 0; r < rows; ++r) {
        widen_row_bf16(x + r * cols, cols, buf);
        select_row(buf, cols, K, order, vals + r * K, idx + r * K);
    }
    free(buf);
    free(order);
    return 0;
}
