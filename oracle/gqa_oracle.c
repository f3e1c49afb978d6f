/*
 * gqa_oracle.c -- plain, slow, fp64 CPU oracle for causal grouped-query
 * attention.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP library,
 * and only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load it.  It shares no code, header, table or helper with the HIP
 * path (causal_grouped_query_amd/csrc) and never includes anything from it.
 *
 * What it computes is the definition itself, written out:
 *
 *   o_a = softmax( Q_a K_{g(a)}^T * scale + M ) V_{g(a)}
 *
 * ("Attention variants" page, section on unified notation, the display
 * equation; the same dense form appears on "Attention Architecture Evolution",
 * section Full Attention / GQA).  For every batch b, query head a and query
 * index i:
 *
 *   1. g = floor(a / (Hq/Hkv))              -- consecutive query heads share
 *                                             one KV head (GQA section;
 *                                             minimal semantic implementation)
 *   2. the query's absolute position is p = Tk_b - Tq + i, where Tk_b is Tk
 *      (forward) or the per-sequence length len_b (decode); a suffix of Tq
 *      queries therefore sits at the end of the key sequence ("Attention
 *      variants", minimal semantic implementation and the section on masks
 *      and incremental positions)
 *   3. visible keys J = {0..p} when causal, else {0..Tk_b-1}; masked keys are
 *      left out of the sum, which is what a -inf additive mask does.  With a
 *      sliding window of w positions (causal only) J = {max(0, p-w+1)..p}:
 *      the w most recent positions, the current one included ("A Visual
 *      Guide to Attention", section on which positions are visible: SWA
 *      keeps direct access to the most recent w positions)
 *   4. s_j = scale * sum_d q[d] k_j[d]
 *   5. two-pass softmax: m = max_J s_j, e_j = exp(s_j - m), l = sum_J e_j,
 *      P_j = e_j / l ("Linear Attention and Sparse Attention" survey, 2.1:
 *      softmax turns scores into a budget that sums to one)
 *   6. o[d'] = sum_J P_j v_j[d'];  lse = m + ln l
 *
 * No tiling, no online rescaling, no fusion: one row at a time, in fp64.
 * Inputs are read in the caller's storage type (bf16 bit patterns, fp32 or
 * fp64) and widened exactly to fp64 before any arithmetic.
 *
 * The only addition not in the pages is oracle_lse_merge(): the exact merge of
 * softmax partials over disjoint key ranges, used by the tests to pin the
 * split-KV decode reading (the merge is a rewrite of step 5 over a partition
 * of J, exact in real arithmetic).
 *
 * Quantised caches: K and V may be stored as FP8 E4M3 codes with one fp32
 * scale per (b, h, t) row (oracle_attention_e4m3kv).  The value an element
 * stands for is decode(code) * scale, the dequantisation of a block-scaled
 * FP8 cache ("Attention Architecture Evolution", DSA section: the indexer
 * keeps FP8 keys with per-block scales; "Attention variants" lists the
 * scale granularity of quantised K/V as a deployment concern).  decode()
 * follows the OCP 8-bit floating point definition of E4M3: sign bit, four
 * exponent bits with bias 7, three mantissa bits; exponent 0 holds the
 * subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN; there are no
 * infinities (largest finite value 448).  The product is formed in fp64,
 * where it is exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2, ORACLE_E4M3 = 3 };

/* A 4-D tensor view: element (b, h, t, d) lives at base[b*s0 + h*s1 + t*s2 + d*s3]. */
typedef struct {
    const void *base;
    long long s0, s1, s2, s3;
    int dtype;
    const float *sc;         /* ORACLE_E4M3: one scale per (b, h, t) */
    long long ss0, ss1, ss2; /* its element strides */
} view4;

/* Value of an OCP FP8 E4M3 code. */
static double e4m3_value(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    /* normal: (1 + m/8) * 2^(e-7) = (8 + m) * 2^(e-10); subnormal: m * 2^-9 */
    double mag = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return sign ? -mag : mag;
}

static double widen(const view4 *v, int b, int h, int t, int d)
{
    long long idx = (long long)b * v->s0 + (long long)h * v->s1 + (long long)t * v->s2 +
                    (long long)d * v->s3;
    if (v->dtype == ORACLE_BF16) {
        /* bf16 is the upper half of an IEEE binary32; widening is exact */
        uint32_t u = (uint32_t)((const uint16_t *)v->base)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (v->dtype == ORACLE_F32)
        return (double)((const float *)v->base)[idx];
    if (v->dtype == ORACLE_E4M3) {
        double s = (double)v->sc[(long long)b * v->ss0 + (long long)h * v->ss1 + (long long)t * v->ss2];
        return e4m3_value(((const uint8_t *)v->base)[idx]) * s;
    }
    return ((const double *)v->base)[idx];
}

typedef struct {
    view4 q, k, v;
    const int *kv_lens; /* NULL: every sequence has Tk keys */
    int B, Hq, Hkv, Tq, Tk, Dk, Dv;
    double scale;
    int causal;
    int window; /* 0: none; w > 0 (causal only): keys p-w+1 .. p */
    int shard;  /* keys are a shard at other absolute positions: query i sits */
    long long q_minus_k; /* at key index q_minus_k + i of this shard */
} problem;

/* Visible keys of query i of batch b: j in [*lo, return value). */
static int visible_range(const problem *P, int b, int i, int *lo)
{
    int tk_b = P->kv_lens ? P->kv_lens[b] : P->Tk;
    if (tk_b > P->Tk) tk_b = P->Tk;
    if (tk_b < 0) tk_b = 0;
    *lo = 0;
    if (!P->causal) return tk_b;
    /* absolute query position, counted in keys of this array */
    long long pos = P->shard ? P->q_minus_k + i : (long long)tk_b - P->Tq + i;
    long long n = pos + 1;                       /* keys 0..pos are visible */
    if (n > tk_b) n = tk_b;
    if (n < 0) n = 0;
    if (P->window > 0) {
        long long first = pos - P->window + 1; /* the w most recent positions */
        if (first > 0) *lo = (int)(first < n ? first : n);
    }
    return (int)n;
}

/*
 * One output row.  s is scratch of at least Tk + Dk doubles.  probs, if
 * non-NULL, receives P_j for j < Tk (zero for masked keys).
 */
static void attend_row(const problem *P, int b, int a, int i, double *s, double *out_row,
                       double *lse_out, double *probs)
{
    int group = P->Hq / P->Hkv;
    int g = a / group; /* step 1: the KV head this query head reads */
    int lo;
    int n = visible_range(P, b, i, &lo); /* steps 2-3: keys lo .. n-1 */

    if (probs)
        for (int j = 0; j < P->Tk; ++j) probs[j] = 0.0;
    if (n <= lo) { /* no visible key: defined as a zero row, lse = -inf */
        for (int d = 0; d < P->Dv; ++d) out_row[d] = 0.0;
        if (lse_out) *lse_out = -INFINITY;
        return;
    }

    /* step 4: scores (the query row is widened once into the scratch tail) */
    double *qrow = s + P->Tk;
    for (int d = 0; d < P->Dk; ++d) qrow[d] = widen(&P->q, b, a, i, d);
    for (int j = lo; j < n; ++j) {
        double acc = 0.0;
        for (int d = 0; d < P->Dk; ++d) acc += qrow[d] * widen(&P->k, b, g, j, d);
        s[j] = P->scale * acc;
    }

    /* step 5: first pass for the max, second for the exponentials */
    double m = s[lo];
    for (int j = lo + 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int j = lo; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int j = lo; j < n; ++j) s[j] /= l; /* s now holds P_j */
    if (probs)
        for (int j = lo; j < n; ++j) probs[j] = s[j];

    /* step 6: weighted sum of values */
    for (int d = 0; d < P->Dv; ++d) {
        double acc = 0.0;
        for (int j = lo; j < n; ++j) acc += s[j] * widen(&P->v, b, g, j, d);
        out_row[d] = acc;
    }
    if (lse_out) *lse_out = m + log(l);
}

static int check_problem(const problem *P)
{
    if (P->B <= 0 || P->Hq <= 0 || P->Hkv <= 0 || P->Tq <= 0 || P->Tk <= 0 || P->Dk <= 0 ||
        P->Dv <= 0)
        return -1;
    if (P->Hq % P->Hkv != 0) return -1;
    if (P->causal && !P->kv_lens && !P->shard && P->Tq > P->Tk) return -1;
    if (P->window < 0 || (P->window > 0 && !P->causal)) return -1;
    return 0;
}

static view4 make_view(const void *base, const long long *st, int dtype)
{
    view4 v;
    v.base = base;
    v.s0 = st[0];
    v.s1 = st[1];
    v.s2 = st[2];
    v.s3 = st[3];
    v.dtype = dtype;
    v.sc = NULL;
    v.ss0 = v.ss1 = v.ss2 = 0;
    return v;
}

/*
 * Attention over every row, or over a list of rows.
 *
 * q, k, v: base pointers with element strides qs/ks/vs[4] over (b, h, t, d)
 * and storage types q_dt/k_dt/v_dt (0 bf16 bits, 1 fp32, 2 fp64).
 * kv_lens: NULL, or B per-sequence key counts (decode caches; keys at
 * positions >= len_b are never read).
 * window: 0, or (with causal) the sliding-window width w >= 1.
 * out: fp64, contiguous [nrows, Dv] when rows != NULL, else [B, Hq, Tq, Dv].
 * lse: NULL or fp64 [nrows] / [B, Hq, Tq] (natural log).
 * rows: NULL, or nrows flattened row ids r = ((b*Hq) + a)*Tq + i.
 * Returns 0, or -1 for an inconsistent problem.
 */
static int run_rows(const problem *P, const long long *rows, long long nrows, double *out,
                    double *lse, int nthreads);

int oracle_attention(const void *q, const long long *qs, int q_dt, const void *k,
                     const long long *ks, int k_dt, const void *v, const long long *vs,
                     int v_dt, const int *kv_lens, int B, int Hq, int Hkv, int Tq, int Tk,
                     int Dk, int Dv, double scale, int causal, int window, const long long *rows,
                     long long nrows, double *out, double *lse, int nthreads)
{
    problem P = {0};
    P.q = make_view(q, qs, q_dt);
    P.k = make_view(k, ks, k_dt);
    P.v = make_view(v, vs, v_dt);
    P.kv_lens = kv_lens;
    P.B = B;
    P.Hq = Hq;
    P.Hkv = Hkv;
    P.Tq = Tq;
    P.Tk = Tk;
    P.Dk = Dk;
    P.Dv = Dv;
    P.scale = scale;
    P.causal = causal;
    P.window = window;
    if (check_problem(&P)) return -1;
    return run_rows(&P, rows, nrows, out, lse, nthreads);
}

/* Every row, or the listed rows, of a checked problem. */
static int run_rows(const problem *P, const long long *rows, long long nrows, double *out,
                    double *lse, int nthreads)
{
    const int B = P->B, Hq = P->Hq, Tq = P->Tq, Tk = P->Tk, Dk = P->Dk, Dv = P->Dv;
    long long total = rows ? nrows : (long long)B * Hq * Tq;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * ((size_t)Tk + (size_t)Dk));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (long long r = 0; r < total; ++r) {
                long long id = rows ? rows[r] : r;
                if (id < 0 || id >= (long long)B * Hq * Tq) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                int i = (int)(id % Tq);
                int a = (int)((id / Tq) % Hq);
                int b = (int)(id / ((long long)Tq * Hq));
                attend_row(P, b, a, i, s, out + r * Dv, lse ? lse + r : NULL, NULL);
            }
            free(s);
        }
    }
    return bad ? -1 : 0;
}

/* The probability row P_j (j < Tk, zero where masked) of one (b, a, i). */
int oracle_probs(const void *q, const long long *qs, int q_dt, const void *k,
                 const long long *ks, int k_dt, const void *v, const long long *vs, int v_dt,
                 const int *kv_lens, int B, int Hq, int Hkv, int Tq, int Tk, int Dk, int Dv,
                 double scale, int causal, int window, int b, int a, int i, double *probs,
                 double *out_row)
{
    problem P = {0};
    P.q = make_view(q, qs, q_dt);
    P.k = make_view(k, ks, k_dt);
    P.v = make_view(v, vs, v_dt);
    P.kv_lens = kv_lens;
    P.B = B;
    P.Hq = Hq;
    P.Hkv = Hkv;
    P.Tq = Tq;
    P.Tk = Tk;
    P.Dk = Dk;
    P.Dv = Dv;
    P.scale = scale;
    P.causal = causal;
    P.window = window;
    if (check_problem(&P) || b < 0 || b >= B || a < 0 || a >= Hq || i < 0 || i >= Tq) return -1;
    double *s = (double *)malloc(sizeof(double) * ((size_t)Tk + (size_t)Dk));
    if (!s) return -1;
    attend_row(&P, b, a, i, s, out_row, NULL, probs);
    free(s);
    return 0;
}

/*
 * Exact merge of softmax partials over disjoint key ranges.
 * o_parts: [S, R, Dv] per-part normalised outputs; lse_parts: [S, R] natural
 * log-sum-exp of each part (-inf for an empty part).  Writes out [R, Dv] and
 * lse [R]:  L = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - L) o_s.
 */
void oracle_lse_merge(const double *o_parts, const double *lse_parts, int S, long long R, int Dv,
                      double *out, double *lse)
{
    for (long long r = 0; r < R; ++r) {
        double m = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (lse_parts[(long long)s * R + r] > m) m = lse_parts[(long long)s * R + r];
        if (m == -INFINITY) {
            for (int d = 0; d < Dv; ++d) out[r * Dv + d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double z = 0.0;
        for (int s = 0; s < S; ++s) z += exp(lse_parts[(long long)s * R + r] - m);
        double L = m + log(z);
        for (int d = 0; d < Dv; ++d) {
            double acc = 0.0;
            for (int s = 0; s < S; ++s) {
                double w = exp(lse_parts[(long long)s * R + r] - L);
                if (w != 0.0) acc += w * o_parts[((long long)s * R + r) * Dv + d];
            }
            out[r * Dv + d] = acc;
        }
        lse[r] = L;
    }
}

/*
 * oracle_attention over a quantised cache: k and v hold E4M3 codes (one byte
 * each, element strides ks / vs), k_scale / v_scale one fp32 scale per
 * (b, h, t) with element strides kss / vss[3].  q is read as for
 * oracle_attention (q_dt).
 */
int oracle_attention_e4m3kv(const void *q, const long long *qs, int q_dt, const void *k,
                            const long long *ks, const float *k_scale, const long long *kss,
                            const void *v, const long long *vs, const float *v_scale,
                            const long long *vss, const int *kv_lens, int B, int Hq, int Hkv,
                            int Tq, int Tk, int Dk, int Dv, double scale, int causal,
                            const long long *rows, long long nrows, double *out, double *lse,
                            int nthreads)
{
    problem P = {0};
    P.q = make_view(q, qs, q_dt);
    P.k = make_view(k, ks, ORACLE_E4M3);
    P.v = make_view(v, vs, ORACLE_E4M3);
    if (!k_scale || !v_scale) return -1;
    P.k.sc = k_scale;
    P.k.ss0 = kss[0];
    P.k.ss1 = kss[1];
    P.k.ss2 = kss[2];
    P.v.sc = v_scale;
    P.v.ss0 = vss[0];
    P.v.ss1 = vss[1];
    P.v.ss2 = vss[2];
    P.kv_lens = kv_lens;
    P.B = B;
    P.Hq = Hq;
    P.Hkv = Hkv;
    P.Tq = Tq;
    P.Tk = Tk;
    P.Dk = Dk;
    P.Dv = Dv;
    P.scale = scale;
    P.causal = causal;
    P.window = 0;
    if (check_problem(&P)) return -1;
    return run_rows(&P, rows, nrows, out, lse, nthreads);
}

/*
 * Attention of Tq queries over one shard of the keys (context / sequence
 * parallelism: each device holds a slice of the key axis and produces a
 * partial result to be merged with oracle_lse_merge).  Query i sits at
 * absolute position q_pos0 + i, key j of the shard at k_pos0 + j; with
 * causal, key j is visible iff k_pos0 + j <= q_pos0 + i.  A query that sees
 * no key of the shard gets a zero row and lse = -inf.  Other arguments as
 * for oracle_attention (no kv_lens, no window).
 */
int oracle_attention_shard(const void *q, const long long *qs, int q_dt, const void *k,
                           const long long *ks, int k_dt, const void *v, const long long *vs,
                           int v_dt, int B, int Hq, int Hkv, int Tq, int Tk, int Dk, int Dv,
                           double scale, int causal, long long q_pos0, long long k_pos0,
                           const long long *rows, long long nrows, double *out, double *lse,
                           int nthreads)
{
    problem P = {0};
    P.q = make_view(q, qs, q_dt);
    P.k = make_view(k, ks, k_dt);
    P.v = make_view(v, vs, v_dt);
    P.kv_lens = NULL;
    P.B = B;
    P.Hq = Hq;
    P.Hkv = Hkv;
    P.Tq = Tq;
    P.Tk = Tk;
    P.Dk = Dk;
    P.Dv = Dv;
    P.scale = scale;
    P.causal = causal;
    P.window = 0;
    P.shard = 1;
    P.q_minus_k = q_pos0 - k_pos0;
    if (check_problem(&P)) return -1;
    return run_rows(&P, rows, nrows, out, lse, nthreads);
}

/* The 256 E4M3 code values (for checking the decoder). */
void oracle_e4m3_table(double *out)
{
    for (int c = 0; c < 256; ++c) out[c] = e4m3_value((uint8_t)c);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
