/*
 * oracle_check.c -- drives every entry point of oracle/gqa_oracle.c on small
 * seeded problems, built with AddressSanitizer and UndefinedBehaviorSanitizer
 * by tests/test_sanitizers_cpu.py.  Besides running clean under the
 * sanitizers, each call is checked against a property the definition fixes:
 * finite results, probability rows that sum to 1 and reproduce the output
 * row, an exact merge of two key halves, the E4M3 code table's anchors, and
 * the rejection of an inconsistent problem.  Exit status 0 iff all hold.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention(const void *q, const long long *qs, int q_dt, const void *k, const long long *ks, int k_dt,
                     const void *v, const long long *vs, int v_dt, const int *kv_lens, int B, int Hq, int Hkv,
                     int Tq, int Tk, int Dk, int Dv, double scale, int causal, int window, const long long *rows,
                     long long nrows, double *out, double *lse, int nthreads);
int oracle_probs(const void *q, const long long *qs, int q_dt, const void *k, const long long *ks, int k_dt,
                 const void *v, const long long *vs, int v_dt, const int *kv_lens, int B, int Hq, int Hkv, int Tq,
                 int Tk, int Dk, int Dv, double scale, int causal, int window, int b, int a, int i, double *probs,
                 double *out_row);
void oracle_lse_merge(const double *o_parts, const double *lse_parts, int S, long long R, int Dv, double *out,
                      double *lse);
int oracle_attention_e4m3kv(const void *q, const long long *qs, int q_dt, const void *k, const long long *ks,
                            const float *k_scale, const long long *kss, const void *v, const long long *vs,
                            const float *v_scale, const long long *vss, const int *kv_lens, int B, int Hq, int Hkv,
                            int Tq, int Tk, int Dk, int Dv, double scale, int causal, const long long *rows,
                            long long nrows, double *out, double *lse, int nthreads);
int oracle_attention_shard(const void *q, const long long *qs, int q_dt, const void *k, const long long *ks,
                           int k_dt, const void *v, const long long *vs, int v_dt, int B, int Hq, int Hkv, int Tq,
                           int Tk, int Dk, int Dv, double scale, int causal, long long q_pos0, long long k_pos0,
                           const long long *rows, long long nrows, double *out, double *lse, int nthreads);
void oracle_e4m3_table(double *out);

enum { BF16 = 0, F32 = 1, F64 = 2 };

static unsigned long long rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void)  /* xorshift64*, in [-1, 1) */
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++failures;                                   \
        }                                                 \
    } while (0)

/* contiguous element strides of a [d0, d1, d2, d3] tensor */
static void strides(long long *s, int d1, int d2, int d3)
{
    s[3] = 1;
    s[2] = d3;
    s[1] = (long long)d2 * d3;
    s[0] = (long long)d1 * d2 * d3;
}

static double *randn_f64(size_t n)
{
    double *x = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = uniform();
    return x;
}

int main(void)
{
    const int B = 2, Hq = 4, Hkv = 2, Tq = 5, Tk = 9, Dk = 16, Dv = 8;
    double *q = randn_f64((size_t)B * Hq * Tq * Dk), *k = randn_f64((size_t)B * Hkv * Tk * Dk);
    double *v = randn_f64((size_t)B * Hkv * Tk * Dv);
    long long qs[4], ks[4], vs[4];
    strides(qs, Hq, Tq, Dk);
    strides(ks, Hkv, Tk, Dk);
    strides(vs, Hkv, Tk, Dv);
    const double scale = 0.25;
    double *out = (double *)calloc((size_t)B * Hq * Tq * Dv, sizeof(double));
    double *lse = (double *)calloc((size_t)B * Hq * Tq, sizeof(double));

    /* full causal suffix attention; every probability row sums to 1 and P V is the output row */
    int rc = oracle_attention(q, qs, F64, k, ks, F64, v, vs, F64, NULL, B, Hq, Hkv, Tq, Tk, Dk, Dv, scale, 1, 0,
                              NULL, 0, out, lse, 2);
    CHECK(rc == 0, "attention rc %d", rc);
    for (int b = 0; b < B; ++b)
        for (int a = 0; a < Hq; ++a)
            for (int i = 0; i < Tq; ++i) {
                double probs[9], row[8], sum = 0.0;
                rc = oracle_probs(q, qs, F64, k, ks, F64, v, vs, F64, NULL, B, Hq, Hkv, Tq, Tk, Dk, Dv, scale, 1, 0, b,
                                  a, i, probs, row);
                CHECK(rc == 0, "probs rc %d", rc);
                for (int j = 0; j < Tk; ++j) sum += probs[j];
                CHECK(fabs(sum - 1.0) < 1e-12, "probs sum %.17g", sum);
                for (int j = Tk - Tq + i + 1; j < Tk; ++j) CHECK(probs[j] == 0.0, "future key %d weighted", j);
                const double *o = out + (((size_t)b * Hq + a) * Tq + i) * Dv;
                for (int d = 0; d < Dv; ++d) {
                    double pv = 0.0;
                    for (int j = 0; j < Tk; ++j) pv += probs[j] * v[(((size_t)b * Hkv + a / 2) * Tk + j) * Dv + d];
                    CHECK(fabs(pv - o[d]) < 1e-12 && fabs(row[d] - o[d]) < 1e-12, "row mismatch");
                }
            }

    /* decode rows over per-sequence lengths (one of them 0), a row subset, a window */
    const int lens[2] = {0, 7};
    long long rows[3] = {1, 5, 7};
    double out3[3 * 8], lse3[3];
    long long q1s[4];
    strides(q1s, Hq, 1, Dk);
    rc = oracle_attention(q, q1s, F64, k, ks, F64, v, vs, F64, lens, B, Hq, Hkv, 1, Tk, Dk, Dv, scale, 1, 0, rows, 3,
                          out3, lse3, 1);
    CHECK(rc == 0, "decode rc %d", rc);
    CHECK(out3[0] == 0.0 && isinf(lse3[0]) && lse3[0] < 0, "empty sequence row");
    for (int r = 1; r < 3; ++r) CHECK(isfinite(lse3[r]), "decode lse");
    rc = oracle_attention(q, qs, F64, k, ks, F64, v, vs, F64, NULL, B, Hq, Hkv, Tq, Tk, Dk, Dv, scale, 1, 3, NULL, 0,
                          out, lse, 2);
    CHECK(rc == 0, "window rc %d", rc);

    /* merge of the two key halves of a shard split equals the whole */
    double *o_parts = (double *)malloc(sizeof(double) * 2 * B * Hq * Tq * Dv);
    double *l_parts = (double *)malloc(sizeof(double) * 2 * B * Hq * Tq);
    const long long R = (long long)B * Hq * Tq;
    long long kh[4] = {ks[0], ks[1], ks[2], ks[3]}, vh[4] = {vs[0], vs[1], vs[2], vs[3]};
    rc = oracle_attention_shard(q, qs, F64, k, kh, F64, v, vh, F64, B, Hq, Hkv, Tq, 4, Dk, Dv, scale, 1, 4, 0, NULL,
                                0, o_parts, l_parts, 2);
    CHECK(rc == 0, "shard 0 rc %d", rc);
    rc = oracle_attention_shard(q, qs, F64, k + 4 * Dk, kh, F64, v + 4 * Dv, vh, F64, B, Hq, Hkv, Tq, 5, Dk, Dv,
                                scale, 1, 4, 4, NULL, 0, o_parts + R * Dv, l_parts + R, 2);
    CHECK(rc == 0, "shard 1 rc %d", rc);
    double *merged = (double *)malloc(sizeof(double) * R * Dv), *mlse = (double *)malloc(sizeof(double) * R);
    oracle_lse_merge(o_parts, l_parts, 2, R, Dv, merged, mlse);
    rc = oracle_attention(q, qs, F64, k, ks, F64, v, vs, F64, NULL, B, Hq, Hkv, Tq, Tk, Dk, Dv, scale, 1, 0, NULL, 0,
                          out, lse, 2);
    for (long long r = 0; r < R; ++r) {
        CHECK(fabs(mlse[r] - lse[r]) < 1e-12, "merged lse");
        for (int d = 0; d < Dv; ++d) CHECK(fabs(merged[r * Dv + d] - out[r * Dv + d]) < 1e-12, "merged output");
    }

    /* E4M3: table anchors, and a small FP8-cache problem */
    double table[256];
    oracle_e4m3_table(table);
    CHECK(table[0x38] == 1.0 && table[0x7E] == 448.0 && table[0x01] == ldexp(1.0, -9) && isnan(table[0x7F]),
          "e4m3 anchors");
    unsigned char *kc = (unsigned char *)malloc((size_t)B * Hkv * Tk * Dk), *vc = (unsigned char *)malloc(
        (size_t)B * Hkv * Tk * Dv);
    for (size_t i = 0; i < (size_t)B * Hkv * Tk * Dk; ++i) kc[i] = (unsigned char)((i * 37) % 0x7E);
    for (size_t i = 0; i < (size_t)B * Hkv * Tk * Dv; ++i) vc[i] = (unsigned char)((i * 53) % 0x7E);
    float *ksc = (float *)malloc(sizeof(float) * B * Hkv * Tk), *vsc = (float *)malloc(sizeof(float) * B * Hkv * Tk);
    for (int i = 0; i < B * Hkv * Tk; ++i) {
        ksc[i] = 0.01f;
        vsc[i] = 0.02f;
    }
    long long kss[3] = {(long long)Hkv * Tk, Tk, 1};
    rc = oracle_attention_e4m3kv(q, q1s, F64, kc, ks, ksc, kss, vc, vs, vsc, kss, lens, B, Hq, Hkv, 1, Tk, Dk, Dv,
                                 scale, 1, NULL, 0, out, lse, 2);
    CHECK(rc == 0, "e4m3 rc %d", rc);
    for (long long r = Hq; r < 2 * Hq; ++r) CHECK(isfinite(lse[r]), "e4m3 lse");

    /* an inconsistent problem is rejected */
    rc = oracle_attention(q, qs, F64, k, ks, F64, v, vs, F64, NULL, B, 3, Hkv, Tq, Tk, Dk, Dv, scale, 1, 0, NULL, 0,
                          out, lse, 1);
    CHECK(rc == -1, "Hq %% Hkv != 0 accepted");

    free(q); free(k); free(v); free(out); free(lse); free(o_parts); free(l_parts); free(merged); free(mlse);
    free(kc); free(vc); free(ksc); free(vsc);
    if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
    else printf("oracle checks passed\n");
    return failures ? 1 : 0;
}
