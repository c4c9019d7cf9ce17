/*
 * attn_oracle.c -- plain, slow, double-precision CPU oracle for causal
 * multi-head scaled dot-product attention with grouped KV heads, and for the
 * rotary position embedding applied to queries and keys.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file:
 * only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no source, header, table or helper with the
 * HIP library, and it is written for a reader who checks it against the
 * pages by eye: every loop follows the formula it cites, in the formula's
 * order, with no blocking, fusion or reordering.
 *
 * Sources (page title -- section):
 *   [P1] "Transformer Math and Implementation Deep Dive" -- Attention Shapes,
 *        Attention Equation, Causal Masking.
 *   [P2] "The Transformer architecture" -- Scaled dot-product attention;
 *        Softmax is a differentiable allocation; Now: RoPE (apply_rope);
 *        What else the modern decoder-only model changed (GQA); Hands-on
 *        (queries of a cached step sit at cache.pos + i).
 *   [P4] "Transformer" (ai-notes) -- Scaled dot-product attention
 *        (Attn(Q,K,V;M)); What is the causal mask?; RoPE (Rotary Positional
 *        Embedding) (theta_i(pos)).
 *
 * Layouts (all row-major, last index fastest, element type double):
 *   q, o : [B][Hq ][Tq][d]        k, v : [B][Hkv][Tk][d]
 *   lse  : [B][Hq][Tq]  (optional, may be NULL)
 *
 * Every function returns 0 on success and a negative value when its
 * arguments cannot describe a defined result (see each function).
 */
#include <math.h>
#include <stdlib.h>

/* Query head hq reads key/value head hq / (Hq / Hkv): contiguous groups of
 * n_rep = Hq / Hkv query heads share one K/V head [P1 Attention Shapes: the
 * K/V heads are repeated or mapped over groups of query heads; P2 GQA: a
 * group of n_rep consecutive query heads reads a single K/V head]. */
static long kv_head_of(long hq, long Hq, long Hkv) { return hq / (Hq / Hkv); }

/* Last key a query row may read.  Causal: key j is visible to query row i
 * iff j <= q_offset + i, where q_offset is the absolute position of the
 * first query row (0 for a plain prefill; cache.pos for a cached step)
 * [P1 Causal Masking: scores[i,j] = -inf if j > i; P4 What is the causal
 * mask?: M[t,s] = 0 for s <= t, -inf otherwise; P2 Hands-on: query
 * positions start at cache.pos + i, keys run from 0 to cache.pos + T - 1].
 * Keys past Tk - 1 do not exist.  Returns -1 when no key is visible. */
static long last_visible_key(long i, long Tk, int causal, long q_offset) {
    if (!causal) return Tk - 1;
    long lim = q_offset + i;
    return lim < Tk - 1 ? lim : Tk - 1;
}

/* One output row o[b,hq,i,:] of
 *     o_i = sum_j alpha_ij v_j,
 *     alpha_ij = exp(s_ij) / sum_j' exp(s_ij'),   s_ij = scale * q_i . k_j
 * over the visible keys j [P2 Scaled dot-product attention; P4 Attn(Q,K,V;M)
 * = softmax(QK^T/sqrt(d_k) + M) V].  A key with M = -inf has exp(-inf) = 0
 * and contributes nothing [P3 "Grasping Codes and Math 02" -- Why Fill with
 * Negative Infinity?], so the masked keys are simply left out of both sums.
 * Subtracting the row maximum m from every score before exp leaves alpha
 * unchanged in exact arithmetic (the factor exp(-m) cancels) and keeps
 * exp() finite.  q and k rows have dk channels, v and o rows dv [P2 Scaled
 * dot-product attention: queries and keys share d_k, values have their own
 * d_v].  `srow` is caller scratch of at least Tk doubles. */
static void attn_row(const double* qi, const double* kh, const double* vh,
                     double* oi, double* lse_i, double* srow,
                     long Tk, long dk, long dv, double scale, long lim) {
    /* scores s_j = scale * sum_c q[c] k[j][c] */
    for (long j = 0; j <= lim; ++j) {
        const double* kj = kh + j * dk;
        double dot = 0.0;
        for (long c = 0; c < dk; ++c) dot += qi[c] * kj[c];
        srow[j] = scale * dot;
    }
    (void)Tk;
    /* m = max_j s_j */
    double m = srow[0];
    for (long j = 1; j <= lim; ++j)
        if (srow[j] > m) m = srow[j];
    /* w_j = exp(s_j - m),  l = sum_j w_j */
    double l = 0.0;
    for (long j = 0; j <= lim; ++j) {
        srow[j] = exp(srow[j] - m);
        l += srow[j];
    }
    /* o[c] = sum_j w_j v[j][c] / l */
    for (long c = 0; c < dv; ++c) oi[c] = 0.0;
    for (long j = 0; j <= lim; ++j) {
        const double* vj = vh + j * dv;
        for (long c = 0; c < dv; ++c) oi[c] += srow[j] * vj[c];
    }
    for (long c = 0; c < dv; ++c) oi[c] /= l;
    /* log of the softmax denominator of the unshifted scores */
    if (lse_i) *lse_i = m + log(l);
}

static int check_shape(long B, long Hq, long Hkv, long Tq, long Tk, long d,
                       double scale, int causal, long q_offset) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Tq <= 0 || Tk <= 0 || d <= 0) return -2;
    if (Hq % Hkv != 0) return -2;
    if (!isfinite(scale)) return -6;
    /* a causal row with no visible key has the softmax of all -inf, which is
     * undefined; the first row sees key q_offset, so q_offset >= 0 */
    if (causal && q_offset < 0) return -5;
    return 0;
}

/* Full attention forward with dk channels in q and k and dv in v and o
 * (q, k: [..][dk]; v, o: [..][dv]).  lse may be NULL. */
int oracle_attn_dv(const double* q, const double* k, const double* v, double* o,
                   double* lse, long B, long Hq, long Hkv, long Tq, long Tk,
                   long dk, long dv, double scale, int causal, long q_offset) {
    int st = check_shape(B, Hq, Hkv, Tq, Tk, dk, scale, causal, q_offset);
    if (st) return st;
    if (dv <= 0) return -2;
    const long nrows = B * Hq * Tq;
    int failed = 0;
#pragma omp parallel
    {
        double* srow = (double*)malloc(sizeof(double) * (size_t)Tk);
        if (!srow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long r = 0; r < nrows; ++r) {
                long i = r % Tq, bh = r / Tq, hq = bh % Hq, b = bh / Hq;
                long hk = kv_head_of(hq, Hq, Hkv);
                const double* qi = q + r * dk;
                const double* kh = k + (b * Hkv + hk) * Tk * dk;
                const double* vh = v + (b * Hkv + hk) * Tk * dv;
                long lim = last_visible_key(i, Tk, causal, q_offset);
                attn_row(qi, kh, vh, o + r * dv, lse ? lse + r : NULL, srow,
                         Tk, dk, dv, scale, lim);
            }
            free(srow);
        }
    }
    return failed ? -10 : 0;
}

/* The forward with one head size d for q, k, v and o. */
int oracle_attn(const double* q, const double* k, const double* v, double* o,
                double* lse, long B, long Hq, long Hkv, long Tq, long Tk,
                long d, double scale, int causal, long q_offset) {
    return oracle_attn_dv(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, d, scale, causal, q_offset);
}

/* Gradients of the attention forward (oracle_attn) for an upstream
 * gradient dO = dL/dO: dq = dL/dq, dk = dL/dk, dv = dL/dv, same layouts as
 * q, k, v.  The pages train this operator ([P1] What To Implement: tiny
 * training loop) through the softmax, a differentiable allocation ([P2]
 * Softmax is a differentiable allocation); they print no gradient formulas,
 * so these are the chain rule of the forward definition, row by row:
 *     o_i = sum_j alpha_ij v_j                 ->  dv_j += alpha_ij dO_i,
 *                                                   g_ij  = dO_i . v_j
 *     alpha_i = softmax(s_i)                   ->  ds_ij = sum_k g_ik dalpha_ik/ds_ij
 *         with dalpha_ik/ds_ij = alpha_ik (delta_jk - alpha_ij)
 *                                              ->  ds_ij = alpha_ij (g_ij - sum_k alpha_ik g_ik)
 *     s_ij = scale q_i . k_j (visible j only)  ->  dq_i += scale ds_ij k_j,
 *                                                   dk_j += scale ds_ij q_i.
 * A K/V head accumulates over every query head of its group and every row.
 * Masked keys have alpha = 0 and receive nothing.  Work is split over
 * (batch, K/V head) so each thread owns the dk / dv rows it adds into.
 * Same status codes as oracle_attn. */
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dO,
                    double* dq, double* dk, double* dv, long B, long Hq, long Hkv,
                    long Tq, long Tk, long d, double scale, int causal, long q_offset) {
    int st = check_shape(B, Hq, Hkv, Tq, Tk, d, scale, causal, q_offset);
    if (st) return st;
    const long R = Hq / Hkv;
    int failed = 0;
#pragma omp parallel
    {
        double* alpha = (double*)malloc(sizeof(double) * (size_t)Tk);
        double* g = (double*)malloc(sizeof(double) * (size_t)Tk);
        double* oi = (double*)malloc(sizeof(double) * (size_t)d);
        if (!alpha || !g || !oi) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bk = 0; bk < B * Hkv; ++bk) {
                const long b = bk / Hkv, hk = bk % Hkv;
                const double* kh = k + bk * Tk * d;
                const double* vh = v + bk * Tk * d;
                double* dkh = dk + bk * Tk * d;
                double* dvh = dv + bk * Tk * d;
                for (long x = 0; x < Tk * d; ++x) { dkh[x] = 0.0; dvh[x] = 0.0; }
                for (long hq = hk * R; hq < (hk + 1) * R; ++hq) {
                    for (long i = 0; i < Tq; ++i) {
                        const long r = (b * Hq + hq) * Tq + i;
                        const double* qi = q + r * d;
                        const double* gi = dO + r * d;
                        double* dqi = dq + r * d;
                        const long lim = last_visible_key(i, Tk, causal, q_offset);
                        /* alpha_ij: the forward's softmax weights (attn_row
                         * leaves exp(s_j - m) in its scratch and o_i / l in
                         * oi; divide the weights by l = sum of them) */
                        attn_row(qi, kh, vh, oi, NULL, alpha, Tk, d, d, scale, lim);
                        double l = 0.0;
                        for (long j = 0; j <= lim; ++j) l += alpha[j];
                        for (long j = 0; j <= lim; ++j) alpha[j] /= l;
                        /* dv_j += alpha_ij dO_i;  g_ij = dO_i . v_j */
                        for (long j = 0; j <= lim; ++j) {
                            const double* vj = vh + j * d;
                            double dot = 0.0;
                            for (long c = 0; c < d; ++c) {
                                dvh[j * d + c] += alpha[j] * gi[c];
                                dot += gi[c] * vj[c];
                            }
                            g[j] = dot;
                        }
                        /* ds_ij = alpha_ij (g_ij - sum_k alpha_ik g_ik) */
                        double ag = 0.0;
                        for (long j = 0; j <= lim; ++j) ag += alpha[j] * g[j];
                        for (long c = 0; c < d; ++c) dqi[c] = 0.0;
                        for (long j = 0; j <= lim; ++j) {
                            const double ds = alpha[j] * (g[j] - ag);
                            const double* kj = kh + j * d;
                            for (long c = 0; c < d; ++c) {
                                dqi[c] += scale * ds * kj[c];
                                dkh[j * d + c] += scale * ds * qi[c];
                            }
                        }
                    }
                }
            }
        }
        free(alpha);
        free(g);
        free(oi);
    }
    return failed ? -10 : 0;
}

/* The same rows as oracle_attn, but only the n rows listed in `rows`
 * (triples b, hq, i), written densely to o_rows[n][d] (and lse_rows[n] if
 * not NULL).  Used to check selected rows of workloads too large for the
 * full loop. */
int oracle_attn_rows(const double* q, const double* k, const double* v,
                     const long* rows, long n, double* o_rows, double* lse_rows,
                     long B, long Hq, long Hkv, long Tq, long Tk, long d,
                     double scale, int causal, long q_offset) {
    int st = check_shape(B, Hq, Hkv, Tq, Tk, d, scale, causal, q_offset);
    if (st) return st;
    for (long r = 0; r < n; ++r) {
        long b = rows[3 * r], hq = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || hq < 0 || hq >= Hq || i < 0 || i >= Tq) return -2;
    }
    int failed = 0;
#pragma omp parallel
    {
        double* srow = (double*)malloc(sizeof(double) * (size_t)Tk);
        if (!srow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (long r = 0; r < n; ++r) {
                long b = rows[3 * r], hq = rows[3 * r + 1], i = rows[3 * r + 2];
                long hk = kv_head_of(hq, Hq, Hkv);
                const double* qi = q + ((b * Hq + hq) * Tq + i) * d;
                const double* kh = k + (b * Hkv + hk) * Tk * d;
                const double* vh = v + (b * Hkv + hk) * Tk * d;
                long lim = last_visible_key(i, Tk, causal, q_offset);
                attn_row(qi, kh, vh, o_rows + r * d,
                         lse_rows ? lse_rows + r : NULL, srow, Tk, d, d, scale, lim);
            }
            free(srow);
        }
    }
    return failed ? -10 : 0;
}

/* Rotary position embedding, in place on x[B][H][T][d].
 *
 * Token t sits at absolute position pos = pos0 + t (pos0 = cache.pos for a
 * cached step [P2 Hands-on: the RoPE angles are taken from cache.pos onward]).  Channel
 * pair p (p = 0 .. d/2 - 1) turns by the angle
 *     theta_p(pos) = pos * base^(-2p/d)
 * [P4 RoPE: theta_i(pos) = pos * 10000^(-2i/d_head)], through the 2x2
 * rotation [[cos, -sin], [sin, cos]] [P2 Now: RoPE, R_m; P4 RoPE].
 *
 * pairing 0 (split-half): pair p is channels (p, p + d/2) [P2 Now: RoPE,
 *     apply_rope: x1, x2 = the two halves; (x1 cos - x2 sin, x1 sin + x2 cos)].
 * pairing 1 (adjacent):   pair p is channels (2p, 2p + 1) [P4 RoPE].
 * The two differ by a channel permutation [P2 Now: RoPE, warning note].
 *
 * Angle, cosine and sine are taken in double precision.  Returns -4 for an
 * odd d, -2 for other bad sizes. */
int oracle_rope(double* x, long B, long H, long T, long d, long pos0,
                double base, int pairing) {
    if (B <= 0 || H <= 0 || T <= 0 || d <= 0) return -2;
    if (d % 2 != 0) return -4;
    if (pairing != 0 && pairing != 1) return -3;
    if (!(base > 0.0) || !isfinite(base)) return -6;
    const long half = d / 2;
    const long nvec = B * H * T;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < nvec; ++r) {
        long t = r % T;
        double pos = (double)(pos0 + t);
        double* xr = x + r * d;
        for (long p = 0; p < half; ++p) {
            double theta = pos * pow(base, -2.0 * (double)p / (double)d);
            double cs = cos(theta), sn = sin(theta);
            long a = pairing == 0 ? p : 2 * p;
            long b2 = pairing == 0 ? p + half : 2 * p + 1;
            double x1 = xr[a], x2 = xr[b2];
            xr[a] = x1 * cs - x2 * sn;
            xr[b2] = x1 * sn + x2 * cs;
        }
    }
    return 0;
}

/* RoPE angle table: for positions pos0 .. pos0 + T - 1 and pairs
 * p = 0 .. d/2 - 1, the cosine and sine of theta_p(pos) = pos * base^(-2p/d)
 * [P4 RoPE], taken in double precision exactly as oracle_rope takes them and
 * then rounded once to float32 (the precision the rotation tables are stored
 * in).  out: float [T][d/2][2], (cos, sin).  Returns -4 for an odd d, -2 for
 * other bad sizes, -6 for a bad base. */
int oracle_rope_table(float* out, long T, long d, long pos0, double base) {
    if (T <= 0 || d <= 0 || pos0 < 0) return -2;
    if (d % 2 != 0) return -4;
    if (!(base > 0.0) || !isfinite(base)) return -6;
    const long half = d / 2;
    for (long t = 0; t < T; ++t) {
        const double position = (double)(pos0 + t);
        for (long p = 0; p < half; ++p) {
            const double theta = position * pow(base, -(2.0 * (double)p) / (double)d);
            out[(t * half + p) * 2 + 0] = (float)cos(theta);
            out[(t * half + p) * 2 + 1] = (float)sin(theta);
        }
    }
    return 0;
}
