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
 *   [ATTN]   the paper summary, section 7.1: O = softmax(Q K^T) V row by row
 *            (the logits X = Q K^T, A = softmax(X) over each row, O = A V),
 *            with the scale 1/sqrt(d) and the causal mask (key j visible to
 *            query i when j <= i) of "6.2 FlashAttention V2 chi tiết",
 *            sections 5.1 and 6.1, and the per-row logsumexp L = m + log(l)
 *            of its section 7.1.
 *   [TILED]  the paper summary, section 7.2.3 (the tiled recurrence of
 *            (m, d', o')) in the delayed-rescaling form of "6.2 FlashAttention
 *            V2 chi tiết", sections 3.2 and 6.1: per tile of b keys,
 *            m_new = max(m, rowmax S), l = e^{m - m_new} l + rowsum e^{S - m_new},
 *            o~ = e^{m - m_new} o~ + e^{S - m_new} V, and O = o~ / l at the end.
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
 *   - Attention takes bf16 Q, K, V (widened exactly) laid out [heads, n, d],
 *     logits s_ij = scale * sum_k Q[i,k] K[j,k] in double; `scale` is passed
 *     in (1/sqrt(d) on the pages).  The causal mask needs as many queries as
 *     keys and hides key j from query i when j > i, so no row is fully
 *     masked.  `oabs` (optional) receives sum_j a_ij |V[j,:]|, the same
 *     weights on |V|: the scale of the rounding error of O.
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

/* ---------------------------------------------------------------------- */
/* [ATTN] O = softmax(scale * Q K^T) V, row by row, by the definition:     */
/* the row of logits, its maximum, the sum of e^{s - m}, the weights       */
/* a_j = e^{s_j - m} / l, then O[i,:] = sum_j a_j V[j,:];                 */
/* L[i] = m + log(l).                                                      */
/* ---------------------------------------------------------------------- */
static void widen_mat_bf16(const uint16_t *src, int64_t n, double *dst)
{
    for (int64_t j = 0; j < n; ++j)
        dst[j] = bf16_bits_to_double(src[j]);
}

/* q [heads, nq, d], k and v [heads, nk, d] (bf16 bits); o [heads, nq, d],
 * lse [heads, nq] and oabs [heads, nq, d] (double; lse and oabs may be NULL).
 * The nq query rows are rows q_off .. q_off + nq - 1 of each head (so a test
 * may take a subset of rows); with `causal`, query row r sees keys j <= r,
 * which needs q_off + nq <= nk.  Returns 0, -1 on allocation failure, -2 for
 * bad sizes. */
int oracle_attention_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t heads, int64_t nq,
                          int64_t nk, int64_t d, double scale, int causal, int64_t q_off, double *o, double *lse,
                          double *oabs)
{
    if (heads < 0 || nq < 0 || nk < 1 || d < 1 || q_off < 0 || (causal && q_off + nq > nk))
        return -2;
    double *qr = (double *)malloc((size_t)d * sizeof(double));
    double *kv = (double *)malloc((size_t)(nk * d) * sizeof(double));
    double *vv = (double *)malloc((size_t)(nk * d) * sizeof(double));
    double *s = (double *)malloc((size_t)nk * sizeof(double));
    double *a = (double *)malloc((size_t)nk * sizeof(double));
    if (!qr || !kv || !vv || !s || !a) {
        free(qr);
        free(kv);
        free(vv);
        free(s);
        free(a);
        return -1;
    }
    for (int64_t h = 0; h < heads; ++h) {
        widen_mat_bf16(k + h * nk * d, nk * d, kv);
        widen_mat_bf16(v + h * nk * d, nk * d, vv);
        for (int64_t i = 0; i < nq; ++i) {
            widen_mat_bf16(q + (h * nq + i) * d, d, qr);
            const int64_t nvis = causal ? q_off + i + 1 : nk; /* keys 0 .. nvis-1 are visible */
            /* logits */
            for (int64_t j = 0; j < nvis; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += qr[c] * kv[j * d + c];
                s[j] = scale * dot;
            }
            /* softmax of the row: maximum, sum, weights */
            double m = -INFINITY;
            for (int64_t j = 0; j < nvis; ++j)
                if (s[j] > m)
                    m = s[j];
            double l = 0.0;
            for (int64_t j = 0; j < nvis; ++j)
                l += exp(s[j] - m);
            for (int64_t j = 0; j < nvis; ++j)
                a[j] = exp(s[j] - m) / l;
            /* O = A V */
            double *orow = o + (h * nq + i) * d;
            double *arow = oabs ? oabs + (h * nq + i) * d : NULL;
            for (int64_t c = 0; c < d; ++c)
                orow[c] = 0.0;
            if (arow)
                for (int64_t c = 0; c < d; ++c)
                    arow[c] = 0.0;
            for (int64_t j = 0; j < nvis; ++j) {
                for (int64_t c = 0; c < d; ++c)
                    orow[c] += a[j] * vv[j * d + c];
                if (arow)
                    for (int64_t c = 0; c < d; ++c)
                        arow[c] += a[j] * fabs(vv[j * d + c]);
            }
            if (lse)
                lse[h * nq + i] = m + log(l);
        }
    }
    free(qr);
    free(kv);
    free(vv);
    free(s);
    free(a);
    return 0;
}

/* [TILED] the same result by the pages' tiled recurrence, tiles of `tile`
 * keys in order, the output kept unnormalised and divided once at the end.
 * The state starts at (m, l, o~) = (-inf, 0, 0).  Same arguments as
 * oracle_attention_bf16 (no oabs). */
int oracle_attention_tiled_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t heads, int64_t nq,
                                int64_t nk, int64_t d, double scale, int causal, int64_t q_off, int64_t tile,
                                double *o, double *lse)
{
    if (heads < 0 || nq < 0 || nk < 1 || d < 1 || tile < 1 || q_off < 0 || (causal && q_off + nq > nk))
        return -2;
    double *qr = (double *)malloc((size_t)d * sizeof(double));
    double *kv = (double *)malloc((size_t)(nk * d) * sizeof(double));
    double *vv = (double *)malloc((size_t)(nk * d) * sizeof(double));
    double *s = (double *)malloc((size_t)tile * sizeof(double));
    double *acc = (double *)malloc((size_t)d * sizeof(double));
    if (!qr || !kv || !vv || !s || !acc) {
        free(qr);
        free(kv);
        free(vv);
        free(s);
        free(acc);
        return -1;
    }
    for (int64_t h = 0; h < heads; ++h) {
        widen_mat_bf16(k + h * nk * d, nk * d, kv);
        widen_mat_bf16(v + h * nk * d, nk * d, vv);
        for (int64_t i = 0; i < nq; ++i) {
            widen_mat_bf16(q + (h * nq + i) * d, d, qr);
            const int64_t nvis = causal ? q_off + i + 1 : nk;
            double m = -INFINITY, l = 0.0;
            for (int64_t c = 0; c < d; ++c)
                acc[c] = 0.0;
            for (int64_t j0 = 0; j0 < nvis; j0 += tile) {
                const int64_t nt = (nvis - j0) < tile ? (nvis - j0) : tile;
                /* the tile's logits and their maximum */
                double m_tile = -INFINITY;
                for (int64_t t = 0; t < nt; ++t) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        dot += qr[c] * kv[(j0 + t) * d + c];
                    s[t] = scale * dot;
                    if (s[t] > m_tile)
                        m_tile = s[t];
                }
                /* rescale the state to the new maximum, then add the tile */
                const double m_new = m > m_tile ? m : m_tile;
                const double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
                double rowsum = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc[c] *= alpha;
                for (int64_t t = 0; t < nt; ++t) {
                    const double p = exp(s[t] - m_new);
                    rowsum += p;
                    for (int64_t c = 0; c < d; ++c)
                        acc[c] += p * vv[(j0 + t) * d + c];
                }
                l = alpha * l + rowsum;
                m = m_new;
            }
            double *orow = o + (h * nq + i) * d;
            for (int64_t c = 0; c < d; ++c)
                orow[c] = acc[c] / l;
            if (lse)
                lse[h * nq + i] = m + log(l);
        }
    }
    free(qr);
    free(kv);
    free(vv);
    free(s);
    free(acc);
    return 0;
}
