/*
 * oracle_harness.c -- drives every function of oracle/attn_oracle.c on small
 * heap arrays of exactly the sizes the layouts state, with valid arguments
 * (ragged sizes, GQA groups, cache offsets, both RoPE pairings) and with
 * arguments each function must reject.  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitize_host.py, so an access
 * past any array, a use of freed memory, a signed overflow or a bad shift
 * in the oracle stops the run.  Exit status 0 when every call behaved.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attn(const double* q, const double* k, const double* v, double* o, double* lse, long B,
                long Hq, long Hkv, long Tq, long Tk, long d, double scale, int causal, long q_offset);
int oracle_attn_dv(const double* q, const double* k, const double* v, double* o, double* lse, long B,
                   long Hq, long Hkv, long Tq, long Tk, long dk, long dv, double scale, int causal,
                   long q_offset);
int oracle_attn_rows(const double* q, const double* k, const double* v, const long* rows, long n,
                     double* o_rows, double* lse_rows, long B, long Hq, long Hkv, long Tq, long Tk,
                     long d, double scale, int causal, long q_offset);
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dO, double* dq,
                    double* dk, double* dv, long B, long Hq, long Hkv, long Tq, long Tk, long d,
                    double scale, int causal, long q_offset);
int oracle_rope(double* x, long B, long H, long T, long d, long pos0, double base, int pairing);
int oracle_rope_table(float* out, long T, long d, long pos0, double base);

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,   \
                    __LINE__, #cond);                                       \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static double* rnd(long n, unsigned* s) {
    double* x = (double*)malloc(sizeof(double) * (size_t)n);
    for (long i = 0; i < n; ++i) {
        *s = *s * 1664525u + 1013904223u;
        x[i] = ((double)(*s >> 8) / 16777216.0) * 2.0 - 1.0;
    }
    return x;
}

static void forward_case(long B, long Hq, long Hkv, long Tq, long Tk, long d, long dv, int causal,
                         long qo, unsigned seed) {
    double* q = rnd(B * Hq * Tq * d, &seed);
    double* k = rnd(B * Hkv * Tk * d, &seed);
    double* v = rnd(B * Hkv * Tk * dv, &seed);
    double* o = (double*)malloc(sizeof(double) * (size_t)(B * Hq * Tq * dv));
    double* lse = (double*)malloc(sizeof(double) * (size_t)(B * Hq * Tq));
    if (dv == d) {
        EXPECT(oracle_attn(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, 0.3, causal, qo) == 0);
        EXPECT(oracle_attn(q, k, v, o, NULL, B, Hq, Hkv, Tq, Tk, d, 0.3, causal, qo) == 0);
        /* every row through oracle_attn_rows gives the same bits */
        long n = B * Hq * Tq;
        long* rows = (long*)malloc(sizeof(long) * (size_t)(3 * n));
        double* orow = (double*)malloc(sizeof(double) * (size_t)(n * d));
        double* lrow = (double*)malloc(sizeof(double) * (size_t)n);
        for (long r = 0; r < n; ++r) {
            rows[3 * r] = r / (Hq * Tq);
            rows[3 * r + 1] = (r / Tq) % Hq;
            rows[3 * r + 2] = r % Tq;
        }
        EXPECT(oracle_attn_rows(q, k, v, rows, n, orow, lrow, B, Hq, Hkv, Tq, Tk, d, 0.3, causal, qo) == 0);
        for (long x = 0; x < n * d; ++x) EXPECT(orow[x] == o[x]);
        rows[3 * (n - 1) + 2] = Tq;   /* a row index past Tq is rejected */
        EXPECT(oracle_attn_rows(q, k, v, rows, n, orow, NULL, B, Hq, Hkv, Tq, Tk, d, 0.3, causal, qo) != 0);
        free(rows); free(orow); free(lrow);
        double* dO = rnd(B * Hq * Tq * d, &seed);
        double* dq = (double*)malloc(sizeof(double) * (size_t)(B * Hq * Tq * d));
        double* dk = (double*)malloc(sizeof(double) * (size_t)(B * Hkv * Tk * d));
        double* dvv = (double*)malloc(sizeof(double) * (size_t)(B * Hkv * Tk * d));
        EXPECT(oracle_attn_bwd(q, k, v, dO, dq, dk, dvv, B, Hq, Hkv, Tq, Tk, d, 0.3, causal, qo) == 0);
        for (long x = 0; x < B * Hkv * Tk * d; ++x) EXPECT(isfinite(dk[x]) && isfinite(dvv[x]));
        free(dO); free(dq); free(dk); free(dvv);
    }
    EXPECT(oracle_attn_dv(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, dv, 0.3, causal, qo) == 0);
    for (long x = 0; x < B * Hq * Tq * dv; ++x) EXPECT(isfinite(o[x]));
    free(q); free(k); free(v); free(o); free(lse);
}

int main(void) {
    /* (B, Hq, Hkv, Tq, Tk, d, dv, causal, q_offset) */
    forward_case(1, 1, 1, 1, 1, 2, 2, 1, 0, 1u);
    forward_case(2, 4, 2, 7, 7, 8, 8, 1, 0, 2u);
    forward_case(1, 6, 2, 5, 13, 4, 4, 1, 8, 3u);        /* chunk at the end of a cache */
    forward_case(1, 3, 3, 9, 4, 6, 6, 0, 0, 4u);         /* no mask, Tq > Tk */
    forward_case(2, 2, 1, 3, 10, 8, 4, 1, 7, 5u);        /* values of their own width */
    forward_case(1, 2, 1, 4, 6, 4, 4, 1, 2147483640L, 6u);   /* offset far past the keys */

    unsigned s = 7u;
    double* x = rnd(2 * 3 * 5 * 8, &s);
    EXPECT(oracle_rope(x, 2, 3, 5, 8, 0, 10000.0, 0) == 0);
    EXPECT(oracle_rope(x, 2, 3, 5, 8, 16383, 10000.0, 1) == 0);
    EXPECT(oracle_rope(x, 2, 3, 5, 7, 0, 10000.0, 0) == -4);
    EXPECT(oracle_rope(x, 2, 3, 5, 8, 0, 10000.0, 2) == -3);
    EXPECT(oracle_rope(x, 2, 3, 5, 8, 0, -1.0, 0) == -6);
    EXPECT(oracle_rope(x, 0, 3, 5, 8, 0, 10000.0, 0) == -2);
    free(x);
    float* tab = (float*)malloc(sizeof(float) * 5 * 4 * 2);
    EXPECT(oracle_rope_table(tab, 5, 8, 100, 10000.0) == 0);
    EXPECT(oracle_rope_table(tab, 5, 7, 100, 10000.0) == -4);
    EXPECT(oracle_rope_table(tab, 5, 8, -1, 10000.0) == -2);
    free(tab);

    /* rejected shapes write nothing and read nothing */
    double one = 1.0;
    EXPECT(oracle_attn(&one, &one, &one, &one, NULL, 1, 3, 2, 1, 1, 1, 1.0, 1, 0) != 0);   /* Hq % Hkv */
    EXPECT(oracle_attn(&one, &one, &one, &one, NULL, 1, 1, 1, 1, 1, 1, NAN, 1, 0) != 0);   /* scale */
    EXPECT(oracle_attn(&one, &one, &one, &one, NULL, 1, 1, 1, 1, 1, 1, 1.0, 1, -1) != 0);  /* offset */
    EXPECT(oracle_attn(&one, &one, &one, &one, NULL, 1, 1, 1, 0, 1, 1, 1.0, 1, 0) != 0);   /* empty */
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("oracle harness: all calls behaved\n");
    return 0;
}
