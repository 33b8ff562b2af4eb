/*
 * oracle.c -- plain, slow, obviously correct CPU reference for fused
 * scaled-dot-product attention.  TEST INFRASTRUCTURE ONLY: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load this
 * library.  The product path never calls it and shares no code with it.
 *
 * Source of every definition: the blog post "从零实现 vLLM (1.3)：如何加速
 * Attention 计算" (section names below are that page's headings).
 *
 * Everything is computed in IEEE double precision with no tiling, no fusion
 * and no reordering beyond what the definitions state.  Inputs arrive as
 * float32 arrays (bf16 inputs are exactly representable in float32 and are
 * upcast exactly); outputs are double.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ------------------------------------------------------------------------ */
/* Softmax variants ("安全 Softmax"的提出 and 在线 Softmax sections).          */
/* ------------------------------------------------------------------------ */

/* Naive softmax, e^{x_i} / sum_j e^{x_j} (section "安全 Softmax"的提出).
 * Kept only as the negative control: it overflows for large inputs. */
void oracle_softmax_naive(const double *x, int64_t n, double *out)
{
    double den = 0.0;
    for (int64_t j = 0; j < n; ++j) den += exp(x[j]);
    for (int64_t i = 0; i < n; ++i) out[i] = exp(x[i]) / den;
}

/* Safe softmax in three passes (section 解决方法): pass 1 finds the maximum m,
 * pass 2 the denominator sum_j e^{x_j - m}, pass 3 the outputs. */
void oracle_softmax_safe3(const double *x, int64_t n, double *out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) if (x[j] > m) m = x[j];          /* pass 1 */
    double den = 0.0;
    for (int64_t j = 0; j < n; ++j) den += exp(x[j] - m);             /* pass 2 */
    for (int64_t i = 0; i < n; ++i) out[i] = exp(x[i] - m) / den;     /* pass 3 */
}

/* Online softmax in two passes (section 在线 Softmax (2-Pass)).  Pass 1 runs
 * the running maximum m_i = max_{j<=i} x_j together with the proxy
 * denominator d'_i = d'_{i-1} e^{m_{i-1}-m_i} + e^{x_i-m_i} (m_0 = -inf,
 * d'_0 = 0).  Pass 2 forms e^{x_i - m_N} / d'_N.  The running sequences are
 * returned so that they can be checked against hand-derived values. */
void oracle_softmax_online2(const double *x, int64_t n, double *m_seq,
                            double *d_seq, double *out)
{
    double m_prev = -INFINITY, d_prev = 0.0;
    for (int64_t i = 0; i < n; ++i) {                                 /* pass 1 */
        double m_i = x[i] > m_prev ? x[i] : m_prev;
        double carry = (d_prev == 0.0) ? 0.0 : d_prev * exp(m_prev - m_i);
        double d_i = carry + exp(x[i] - m_i);
        if (m_seq) m_seq[i] = m_i;
        if (d_seq) d_seq[i] = d_i;
        m_prev = m_i;
        d_prev = d_i;
    }
    for (int64_t i = 0; i < n; ++i) out[i] = exp(x[i] - m_prev) / d_prev;  /* pass 2 */
}

/* ------------------------------------------------------------------------ */
/* Attention.                                                               */
/* ------------------------------------------------------------------------ */

/* One output row O[i,h,:] of softmax(s * q K^T) V over the visible key set
 * J = [0, n_vis), computed the standard way (section 标准实现方法): the
 * logits row X (first step, scaled as in the note under the second step),
 * the safe softmax row A in three passes, then O = A V (third step).
 *   q   : d values of query row i, head h
 *   k,v : key/value rows of this sequence; row j of head g lives at
 *         k + (j * kv_stride) + g*d
 *   x   : scratch of at least n_vis doubles                                  */
static void attn_row(const float *q, const float *k, const float *v,
                     int64_t kv_stride, int g, int d, int64_t n_vis,
                     double scale, double *x, double *o)
{
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (n_vis <= 0) return;                       /* no visible key: zero row */
    /* first step: X row, x_j = s * sum_c q_c k_{j,c} */
    for (int64_t j = 0; j < n_vis; ++j) {
        const float *kj = k + j * kv_stride + (int64_t)g * d;
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)q[c] * (double)kj[c];
        x[j] = scale * acc;
    }
    /* second step: safe softmax in three passes */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j) if (x[j] > m) m = x[j];
    double den = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) den += exp(x[j] - m);
    /* third step: O = A V, with A_j = e^{x_j - m} / den */
    for (int64_t j = 0; j < n_vis; ++j) {
        double a = exp(x[j] - m) / den;
        const float *vj = v + j * kv_stride + (int64_t)g * d;
        for (int c = 0; c < d; ++c) o[c] += a * (double)vj[c];
    }
}

/* Sequence index b with cu[b] <= t < cu[b+1] (cu is an exclusive prefix sum
 * of lengths, as cu_seqlens in the Prefill section). */
static int seq_of(const int32_t *cu, int batch, int64_t t)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* Variable-length attention (Prefill section: q/k/v concatenated over the
 * batch without padding, sequence b's queries are rows cu_q[b]..cu_q[b+1]-1
 * and its keys/values rows cu_k[b]..cu_k[b+1]-1; V shares K's offsets).
 *
 *   q [total_q, hq, d], k/v [total_k, hkv, d] (float32, row-major)
 *   Query head h reads key/value head h / (hq/hkv).
 *   causal != 0: query i of a sequence with Lq queries and Lk keys sits at
 *   absolute position Lk - Lq + i and sees keys j <= Lk - Lq + i (aligned to
 *   the end of the sequence); causal == 0: every key is visible.
 *   rows == NULL: o is [total_q, hq, d], every row computed.
 *   rows != NULL: o is [nrows, d]; rows[r] = t*hq + h selects query token t,
 *   head h.
 *   Returns 0, or -1 on bad arguments.                                       */
int oracle_attn_varlen(const float *q, const float *k, const float *v,
                       double *o, const int32_t *cu_q, const int32_t *cu_k,
                       int batch, int hq, int hkv, int d, double scale,
                       int causal, const int64_t *rows, int64_t nrows,
                       int nthreads)
{
    if (batch <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv) return -1;
    const int group = hq / hkv;
    const int64_t total_q = cu_q[batch];
    int64_t max_lk = 0;
    for (int b = 0; b < batch; ++b) {
        int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
        if (lk > max_lk) max_lk = lk;
    }
    const int64_t n = rows ? nrows : total_q * hq;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(max_lk > 0 ? max_lk : 1));
        if (!x) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n; ++r) {
            if (!x) continue;
            const int64_t flat = rows ? rows[r] : r;
            const int64_t t = flat / hq;
            const int h = (int)(flat % hq);
            double *orow = o + (rows ? r * d : flat * d);
            if (t < 0 || t >= total_q) { for (int c = 0; c < d; ++c) orow[c] = NAN; continue; }
            const int b = seq_of(cu_q, batch, t);
            const int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b];
            const int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
            const int64_t i = t - cu_q[b];
            int64_t n_vis = causal ? (lk - lq + i + 1) : lk;
            if (n_vis > lk) n_vis = lk;
            const int g = h / group;
            attn_row(q + (t * hq + h) * (int64_t)d,
                     k + (int64_t)cu_k[b] * hkv * d, v + (int64_t)cu_k[b] * hkv * d,
                     (int64_t)hkv * d, g, d, n_vis, scale, x, orow);
        }
        free(x);
    }
    return err ? -1 : 0;
}

/* Single-token decode (Decode section): each sequence b has exactly one new
 * query q[b] and attends to every one of its cache_seqlens[b] cached keys
 * (the store of the new token happens first, so that length includes it;
 * with one query the causal flag hides nothing).  K/V are read from the
 * logical per-sequence arrays k/v [total_k, hkv, d] at offsets cu_k, not from
 * a paged pool.  q and o are [batch, hq, d].                                  */
int oracle_attn_decode(const float *q, const float *k, const float *v,
                       double *o, const int32_t *cu_k, int batch, int hq,
                       int hkv, int d, double scale, int nthreads)
{
    if (batch <= 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv) return -1;
    const int group = hq / hkv;
    int64_t max_lk = 0;
    for (int b = 0; b < batch; ++b) {
        int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
        if (lk > max_lk) max_lk = lk;
    }
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(max_lk > 0 ? max_lk : 1));
        if (!x) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < (int64_t)batch * hq; ++r) {
            if (!x) continue;
            const int b = (int)(r / hq), h = (int)(r % hq);
            const int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
            attn_row(q + r * d, k + (int64_t)cu_k[b] * hkv * d,
                     v + (int64_t)cu_k[b] * hkv * d, (int64_t)hkv * d,
                     h / group, d, lk, scale, x, o + r * d);
        }
        free(x);
    }
    return err ? -1 : 0;
}
