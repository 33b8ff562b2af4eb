/* Drives the CPU oracle (oracle/oracle.c, compiled into this program) under
 * AddressSanitizer and UndefinedBehaviorSanitizer on small ragged cases:
 * empty sequences, Lq > Lk, non-causal, a row subset, decode with a zero
 * context.  Test infrastructure only.  Prints "OK" and exits 0 when every
 * output is finite (or zero where no key is visible) and the safe-softmax
 * closed form of [700, 710, 705] holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_softmax_safe3(const double *x, int64_t n, double *out);
void oracle_softmax_online2(const double *x, int64_t n, double *m_seq, double *d_seq, double *out);
int oracle_attn_varlen(const float *q, const float *k, const float *v, double *o, const int32_t *cu_q,
                       const int32_t *cu_k, int batch, int hq, int hkv, int d, double scale, int causal,
                       const int64_t *rows, int64_t nrows, int nthreads);
int oracle_attn_decode(const float *q, const float *k, const float *v, double *o, const int32_t *cu_k,
                       int batch, int hq, int hkv, int d, double scale, int nthreads);

static float frand(uint32_t *s) {
    *s = *s * 1664525u + 1013904223u;
    return (float)((*s >> 8) & 0xFFFF) / 32768.0f - 1.0f;
}

int main(void) {
    int fails = 0;
    const double x[3] = {700.0, 710.0, 705.0};
    double p[3], m[3], dd[3], p2[3];
    oracle_softmax_safe3(x, 3, p);
    oracle_softmax_online2(x, 3, m, dd, p2);
    const double z = 1.0 + exp(-5.0) + exp(-10.0);
    if (fabs(p[1] - 1.0 / z) > 1e-15 || fabs(p2[0] - exp(-10.0) / z) > 1e-15) ++fails;

    /* varlen: Lq = {0, 5, 7, 2}, Lk = {3, 9, 4, 2}; hq 4, hkv 2, d 8 */
    const int B = 4, hq = 4, hkv = 2, d = 8;
    const int32_t cu_q[5] = {0, 0, 5, 12, 14};
    const int32_t cu_k[5] = {0, 3, 12, 16, 18};
    uint32_t seed = 7;
    float *q = malloc(sizeof(float) * 14 * hq * d), *k = malloc(sizeof(float) * 18 * hkv * d);
    float *v = malloc(sizeof(float) * 18 * hkv * d);
    for (int i = 0; i < 14 * hq * d; ++i) q[i] = frand(&seed);
    for (int i = 0; i < 18 * hkv * d; ++i) { k[i] = frand(&seed); v[i] = frand(&seed); }
    double *o = malloc(sizeof(double) * 14 * hq * d);
    for (int causal = 0; causal < 2; ++causal) {
        if (oracle_attn_varlen(q, k, v, o, cu_q, cu_k, B, hq, hkv, d, 0.35, causal, NULL, 0, 2) != 0) ++fails;
        for (int i = 0; i < 14 * hq * d; ++i) if (!isfinite(o[i])) ++fails;
    }
    /* sequence 2 has Lq 7 > Lk 4: under the causal mask its first 3 rows see nothing -> 0 */
    for (int t = 5; t < 8; ++t)
        for (int c = 0; c < hq * d; ++c) if (o[(int64_t)t * hq * d + c] != 0.0) ++fails;
    const int64_t rows[3] = {0, 13 * hq + 3, 6 * hq + 1};
    double orow[3 * 8];
    if (oracle_attn_varlen(q, k, v, orow, cu_q, cu_k, B, hq, hkv, d, 0.35, 1, rows, 3, 1) != 0) ++fails;
    for (int i = 0; i < 3 * d; ++i) if (!isfinite(orow[i])) ++fails;

    /* decode: contexts {3, 0, 9, 6} over the same K/V rows */
    const int32_t cu_d[5] = {0, 3, 3, 12, 18};
    double od[4 * 4 * 8];
    if (oracle_attn_decode(q, k, v, od, cu_d, 4, hq, hkv, d, 0.35, 2) != 0) ++fails;
    for (int i = 0; i < 4 * hq * d; ++i) if (!isfinite(od[i])) ++fails;
    for (int c = 0; c < hq * d; ++c) if (od[1 * hq * d + c] != 0.0) ++fails;

    free(q); free(k); free(v); free(o);
    printf(fails ? "FAIL %d\n" : "OK\n", fails);
    return fails ? 1 : 0;
}
