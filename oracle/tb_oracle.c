/*
 * TokenButler decode-path ORACLE -- test infrastructure only.
 *
 * A plain, slow CPU implementation of what the decode-time hot path
 * computes, written from the method description in "TokenButler" (technical
 * summary, sections "Core architecture" and "Inference strategy"). It
 * accumulates in double precision and applies exactly the storage roundings
 * listed below. Loops over independent outputs (hidden units, query heads,
 * sequences) are spread over OpenMP threads when built with -fopenmp; every
 * output is still computed by one thread in the order written here, so the
 * results do not depend on the thread count. Only the tests, the smoke check and the benchmark's
 * cpu_baseline leg may load this library; the GPU library never does, and the
 * two share no code, header or table.
 *
 * Storage conventions (all arrays row-major, innermost index last):
 *   bf16 / fp16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *   x      [B, E]                bf16   producer-layer hidden state
 *   w1     [Eh, E]               bf16   MLP layer 1 (out x in)
 *   w2     [Nout, Eh]            bf16   MLP layer 2 (out x in), Nout = n_slots*Hq*dp
 *   h      [B, Eh]               bf16   SiLU(x w1^T), rounded to bf16 (RNE)
 *   qhat   [B, n_slots, Hq, dp]  fp32   predicted importance queries
 *   kc, vc [B, Hkv, Lmax, D]     bf16   full (retained) KV cache
 *   wk     [Hkv, dp, D]          bf16   key projection per KV head (out x in)
 *   kp     [B, Hkv, Lmax, dp]    fp16   projected-key cache
 *   scores [B, Hq, Lmax]         fp32   importance scores
 *   idx    [B, Hq, cap]          int32  ascending attended positions
 *   count  [B, Hq]               int32
 *   q      [B, Hq, D]            bf16   decode query
 *   out    [B, Hq, D]            fp32   attention output
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#define _GNU_SOURCE   /* qsort_r */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops use (1 without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* IEEE-754 storage formats, written from their definitions.           */
/* ------------------------------------------------------------------ */

/* bfloat16 = the upper 16 bits of an IEEE binary32. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), expo - 25);  /* 1.frac * 2^(expo-15) */
    return sign ? -mag : mag;
}

/*
 * Round v to the nearest value with `prec` significant bits (including the
 * leading one), smallest normal 2^emin, largest finite maxf; ties go to the
 * even neighbour; results beyond maxf become infinity. One rounding step,
 * taken straight from double precision.
 */
static double round_to_format(double v, int prec, int emin, double maxf)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    frexp(v, &e);                      /* |v| = m 2^e, 0.5 <= m < 1 */
    int q = e - prec;                  /* exponent of one unit in the last place */
    if (q < emin - prec + 1)
        q = emin - prec + 1;           /* subnormal spacing */
    double r = ldexp(nearbyint(ldexp(v, -q)), q);   /* default mode: nearest-even */
    if (fabs(r) > maxf)
        r = v > 0 ? INFINITY : -INFINITY;
    return r;
}

static uint16_t bf16_bits_rne(double v)
{
    double r = round_to_format(v, 8, -126, ldexp(255.0, 120)); /* (2-2^-7) 2^127 */
    float f = (float)r;                /* exact: r has 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static uint16_t f16_bits_rne(double v)
{
    double r = round_to_format(v, 11, -14, 65504.0);
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (isinf(a))
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int e;
    double m = frexp(a, &e);           /* a = m 2^e */
    int ebiased = e - 1 + 15;          /* a = 1.f 2^(e-1) */
    if (ebiased <= 0)                  /* subnormal: a = frac 2^-24 */
        return sign | (uint16_t)(a * 16777216.0);
    uint16_t frac = (uint16_t)((m * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(ebiased << 10) | frac;
}

/* Exported rounding helpers (pinned against numpy / torch casts). */
uint16_t orc_bf16_bits(double v) { return bf16_bits_rne(v); }
uint16_t orc_f16_bits(double v) { return f16_bits_rne(v); }
double orc_bf16_value(uint16_t b) { return bf16_value(b); }
double orc_f16_value(uint16_t b) { return f16_value(b); }

/* ------------------------------------------------------------------ */
/* Query prediction: a lightweight two-layer MLP on the producer        */
/* layer's hidden state ("Core architecture", query prediction).        */
/* ------------------------------------------------------------------ */

/* SiLU(z) = z * logistic(z). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

void orc_predict_queries(const uint16_t *x, const uint16_t *w1, const uint16_t *w2,
                         uint16_t *h_out, float *qhat,
                         int B, int E, int Eh, int Nout)
{
    uint16_t *h = h_out ? h_out : (uint16_t *)malloc(sizeof(uint16_t) * (size_t)B * Eh);
    for (int b = 0; b < B; ++b) {
#pragma omp parallel for schedule(static)
        for (int j = 0; j < Eh; ++j) {
            double z = 0.0;
            for (int i = 0; i < E; ++i)
                z += bf16_value(x[(size_t)b * E + i]) * bf16_value(w1[(size_t)j * E + i]);
            h[(size_t)b * Eh + j] = bf16_bits_rne(silu(z));
        }
#pragma omp parallel for schedule(static)
        for (int n = 0; n < Nout; ++n) {
            double acc = 0.0;
            for (int j = 0; j < Eh; ++j)
                acc += bf16_value(h[(size_t)b * Eh + j]) * bf16_value(w2[(size_t)n * Eh + j]);
            qhat[(size_t)b * Nout + n] = (float)acc;
        }
    }
    if (!h_out)
        free(h);
}

/* ------------------------------------------------------------------ */
/* Key-cache projection into the predictor's low-dimensional space      */
/* ("Core architecture", key projection), done for a batch of tokens    */
/* at a time ("Inference strategy", batching).                          */
/* ------------------------------------------------------------------ */

void orc_project_keys(const uint16_t *kc, const uint16_t *wk, uint16_t *kp,
                      const int *pos0, int ntok,
                      int B, int Hkv, int Lmax, int D, int dp)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hkv; ++j)
            for (int t = pos0[b]; t < pos0[b] + ntok && t < Lmax; ++t) {
                if (t < 0)
                    continue;
                const uint16_t *krow = kc + (((size_t)b * Hkv + j) * Lmax + t) * D;
                for (int c = 0; c < dp; ++c) {
                    const uint16_t *wrow = wk + ((size_t)j * dp + c) * D;
                    double acc = 0.0;
                    for (int i = 0; i < D; ++i)
                        acc += bf16_value(krow[i]) * bf16_value(wrow[i]);
                    kp[(((size_t)b * Hkv + j) * Lmax + t) * dp + c] = f16_bits_rne(acc);
                }
            }
}

/*
 * One decode step's cache append with batched key projection ("Inference
 * strategy": the newest token's key and value join the retained cache;
 * "Optimizations": the key projection runs once per batch of n_p new tokens
 * rather than every step). Per sequence b, with L = ctx_len[b] and
 * P = proj_len[b]:
 *   if 0 <= P <= L < Lmax: the new rows are written at position L of every
 *   KV head, ctx_len[b] = L + 1, and when L + 1 - P >= n_p the keys
 *   [P, L + 1) are projected (orc_project_keys) and proj_len[b] = L + 1;
 *   otherwise (a full cache or lengths out of range) nothing changes for b.
 *   k_new, v_new [B, Hkv, D] bf16; n_p >= 1.
 */
void orc_append_kv(const uint16_t *k_new, const uint16_t *v_new, uint16_t *kc, uint16_t *vc,
                   uint16_t *kp, const uint16_t *wk, int *ctx_len, int *proj_len,
                   int B, int Hkv, int Lmax, int D, int dp, int n_p)
{
    for (int b = 0; b < B; ++b) {
        int L = ctx_len[b], P = proj_len[b];
        if (!(P >= 0 && P <= L && L < Lmax))
            continue;
        for (int j = 0; j < Hkv; ++j) {
            size_t src = ((size_t)b * Hkv + j) * D;
            size_t dst = (((size_t)b * Hkv + j) * Lmax + L) * D;
            memcpy(kc + dst, k_new + src, sizeof(uint16_t) * (size_t)D);
            memcpy(vc + dst, v_new + src, sizeof(uint16_t) * (size_t)D);
        }
        ctx_len[b] = L + 1;
        if (L + 1 - P >= n_p) {
            size_t off = (size_t)b * Hkv * Lmax;
            orc_project_keys(kc + off * D, wk, kp + off * dp, &P, L + 1 - P, 1, Hkv, Lmax, D, dp);
            proj_len[b] = L + 1;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Scoring: importance = predicted query . projected key               */
/* ("Core architecture", scoring). Query head h reads KV head h/g.      */
/* ------------------------------------------------------------------ */

void orc_score(const float *qhat, int n_slots, int slot, const uint16_t *kp,
               const int *proj_len, float *scores,
               int B, int Hq, int Hkv, int Lmax, int dp)
{
    int g = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            const float *qv = qhat + (((size_t)b * n_slots + slot) * Hq + h) * dp;
            int kvh = h / g;
            int P = proj_len[b] < Lmax ? proj_len[b] : Lmax;
            for (int t = 0; t < P; ++t) {
                const uint16_t *kr = kp + (((size_t)b * Hkv + kvh) * Lmax + t) * dp;
                double acc = 0.0;
                for (int c = 0; c < dp; ++c)
                    acc += (double)qv[c] * f16_value(kr[c]);
                scores[((size_t)b * Hq + h) * Lmax + t] = (float)acc;
            }
        }
}

/* ------------------------------------------------------------------ */
/* Fixed-budget selection with neighbour fetching, unioned with the     */
/* sink and the local window ("Inference strategy": the three buffers;  */
/* "Optimizations": neighbour fetching; "Core architecture": selection  */
/* under a fixed budget).                                               */
/* ------------------------------------------------------------------ */

/* Candidate order: higher score first in IEEE totalOrder (so -0 ranks
 * below +0), and among equal scores the lower position first. */

static int score_above(float a, float b)
{
    if (a != b)
        return a > b;
    return !signbit(a) && signbit(b);  /* +0 above -0 */
}

static int cmp_candidates(const void *pa, const void *pb, void *scores)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    const float *s = (const float *)scores;
    float sa = s[a], sb = s[b];
    if (score_above(sa, sb))
        return -1;
    if (score_above(sb, sa))
        return 1;
    return (a > b) - (a < b);
}

/*
 * Per (b, query head):
 *   eligible region E = [S, min(L - W, P)), empty when the bound is <= S;
 *   the important buffer takes min(K, |E|) tokens, filled greedily: visit
 *   the eligible positions in candidate order; each visited centre c brings
 *   c, then c-1, c+1, c-2, c+2, ... up to distance r, skipping positions
 *   outside E or already taken, until the buffer is full;
 *   the attended set is sink [0, min(S, L)) U window [max(0, L - W), L)
 *   U important, written ascending.
 * Returns 0; -1 if some count would exceed cap; -2 if a length is outside
 * [0, Lmax] (that sequence's first count is then -1).
 */
int orc_select(const float *scores, const int *ctx_len, const int *proj_len,
               int B, int Hq, int Lmax, int S, int W, int K, int r,
               int *idx, int *count, int cap)
{
    int status = 0;
    for (int b = 0; b < B; ++b) {
        int L = ctx_len[b];
        int P = proj_len[b];
        if (L < 0 || L > Lmax || P < 0 || P > Lmax) {
            status = -2;
            count[(size_t)b * Hq] = -1;
            continue;
        }
        int e0 = S;
        int e1 = L - W < P ? L - W : P;
        if (e1 < e0)
            e1 = e0;
        int nE = e1 - e0;
        int need = K < nE ? K : nE;
        int over = 0;   /* some head's count exceeded cap */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : over)
        for (int h = 0; h < Hq; ++h) {
            const float *s = scores + ((size_t)b * Hq + h) * Lmax;
            unsigned char *keep = (unsigned char *)calloc((size_t)(L > 0 ? L : 1), 1);
            int *order = (int *)malloc(sizeof(int) * (size_t)(nE > 0 ? nE : 1));

            for (int i = 0; i < nE; ++i)
                order[i] = e0 + i;
            qsort_r(order, (size_t)nE, sizeof(int), cmp_candidates, (void *)s);

            int taken = 0;
            for (int i = 0; i < nE && taken < need; ++i) {
                int c = order[i];
                for (int d = 0; d <= r && taken < need; ++d) {
                    int cand[2] = {c - d, c + d};
                    int nc = d == 0 ? 1 : 2;
                    for (int k = 0; k < nc && taken < need; ++k) {
                        int t = cand[k];
                        if (t < e0 || t >= e1 || keep[t])
                            continue;
                        keep[t] = 1;
                        ++taken;
                    }
                }
            }

            for (int t = 0; t < L && t < S; ++t)
                keep[t] = 1;
            for (int t = L - W < 0 ? 0 : L - W; t < L; ++t)
                keep[t] = 1;

            int n = 0;
            int *dst = idx + ((size_t)b * Hq + h) * cap;
            for (int t = 0; t < L; ++t)
                if (keep[t]) {
                    if (n < cap)
                        dst[n] = t;
                    else
                        over = 1;
                    ++n;
                }
            count[(size_t)b * Hq + h] = n;
            free(order);
            free(keep);
        }
        if (over)
            status = -1;
    }
    return status;
}

/*
 * Neighbour fetching read the other way ("Optimizations", neighbour
 * fetching: the chosen tokens are widened to take in their neighbours; the
 * summary leaves open whether the neighbours count against the budget). Per
 * (b, query head):
 *   eligible region E and need = min(K, |E|) as for orc_select;
 *   the centres are the first `need` eligible positions in candidate order
 *   (descending score under IEEE totalOrder, lower position first on ties);
 *   every position of E within distance r of a centre is attended (the
 *   neighbours come on top of the budget, so up to (2r+1) * need of them);
 *   the attended set is sink U window U that widened set, written ascending.
 * Returns as orc_select.
 */
int orc_select_dilate(const float *scores, const int *ctx_len, const int *proj_len,
                      int B, int Hq, int Lmax, int S, int W, int K, int r,
                      int *idx, int *count, int cap)
{
    int status = 0;
    for (int b = 0; b < B; ++b) {
        int L = ctx_len[b];
        int P = proj_len[b];
        if (L < 0 || L > Lmax || P < 0 || P > Lmax) {
            status = -2;
            count[(size_t)b * Hq] = -1;
            continue;
        }
        int e0 = S;
        int e1 = L - W < P ? L - W : P;
        if (e1 < e0)
            e1 = e0;
        int nE = e1 - e0;
        int need = K < nE ? K : nE;
        int over = 0;   /* some head's count exceeded cap */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : over)
        for (int h = 0; h < Hq; ++h) {
            const float *s = scores + ((size_t)b * Hq + h) * Lmax;
            unsigned char *keep = (unsigned char *)calloc((size_t)(L > 0 ? L : 1), 1);
            int *order = (int *)malloc(sizeof(int) * (size_t)(nE > 0 ? nE : 1));

            for (int i = 0; i < nE; ++i)
                order[i] = e0 + i;
            qsort_r(order, (size_t)nE, sizeof(int), cmp_candidates, (void *)s);

            for (int i = 0; i < need; ++i) {
                int c = order[i];
                for (int t = c - r; t <= c + r; ++t)
                    if (t >= e0 && t < e1)
                        keep[t] = 1;
            }

            for (int t = 0; t < L && t < S; ++t)
                keep[t] = 1;
            for (int t = L - W < 0 ? 0 : L - W; t < L; ++t)
                keep[t] = 1;

            int n = 0;
            int *dst = idx + ((size_t)b * Hq + h) * cap;
            for (int t = 0; t < L; ++t)
                if (keep[t]) {
                    if (n < cap)
                        dst[n] = t;
                    else
                        over = 1;
                    ++n;
                }
            count[(size_t)b * Hq + h] = n;
            free(order);
            free(keep);
        }
        if (over)
            status = -1;
    }
    return status;
}

/*
 * Distillation loss ("Training": the predictor learns from the frozen base
 * model's masked causal attention distribution by minimizing the cross
 * entropy between the teacher's attention logits and the predictor's
 * logits; the loss is evaluated at a subset of R query positions, which
 * makes it O(R L) instead of O(L^2)). Per (b, r, query head h) with
 * position i = pos[b, r] (clamped to [0, Lmax - 1]) and KV head h / g, over
 * the causal tokens t <= i:
 *   teacher logits z_t = scale * q[b, r, h] . k[b, h/g, t]      (bf16 inputs)
 *   student logits s_t = qhat[b, r, h] . kp[b, h/g, t]          (fp32 . fp16)
 *   p = softmax(z);  loss[b, r, h] = -sum_t p_t log softmax(s)_t
 *                                  = logsumexp_t(s_t) - sum_t p_t s_t
 *   q [B, R, Hq, D] bf16, qhat [B, R, Hq, dp] fp32, loss [B, R, Hq] fp32.
 */
void orc_distill_loss(const uint16_t *q, const uint16_t *kc, const float *qhat,
                      const uint16_t *kp, const int *pos, int B, int R, int Hq, int Hkv,
                      int Lmax, int D, int dp, double scale, float *loss)
{
    int g = Hq / Hkv;
    double *z = (double *)malloc(sizeof(double) * (size_t)Lmax);
    double *sl = (double *)malloc(sizeof(double) * (size_t)Lmax);
    for (int b = 0; b < B; ++b)
        for (int r = 0; r < R; ++r) {
            int i = pos[(size_t)b * R + r];
            if (i < 0)
                i = 0;
            if (i > Lmax - 1)
                i = Lmax - 1;
            for (int h = 0; h < Hq; ++h) {
                const uint16_t *qr = q + (((size_t)b * R + r) * Hq + h) * D;
                const float *qh = qhat + (((size_t)b * R + r) * Hq + h) * dp;
                size_t head = (size_t)b * Hkv + h / g;
                double zmax = -INFINITY, smax = -INFINITY;
                for (int t = 0; t <= i; ++t) {
                    const uint16_t *kr = kc + (head * Lmax + t) * D;
                    const uint16_t *kpr = kp + (head * Lmax + t) * dp;
                    double a = 0.0, c = 0.0;
                    for (int d = 0; d < D; ++d)
                        a += bf16_value(qr[d]) * bf16_value(kr[d]);
                    for (int d = 0; d < dp; ++d)
                        c += (double)qh[d] * f16_value(kpr[d]);
                    z[t] = scale * a;
                    sl[t] = c;
                    if (z[t] > zmax)
                        zmax = z[t];
                    if (sl[t] > smax)
                        smax = sl[t];
                }
                double zs = 0.0, ps = 0.0, ss = 0.0;
                for (int t = 0; t <= i; ++t) {
                    double w = exp(z[t] - zmax);
                    zs += w;
                    ps += w * sl[t];
                    ss += exp(sl[t] - smax);
                }
                loss[((size_t)b * R + r) * Hq + h] = (float)(smax + log(ss) - ps / zs);
            }
        }
    free(sl);
    free(z);
}

/* ------------------------------------------------------------------ */
/* Decode attention over the attended positions only ("Significance":  */
/* the full cache is kept, only the most relevant tokens are read).     */
/* ------------------------------------------------------------------ */

void orc_sparse_attention(const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                          const int *idx, const int *count, int cap,
                          int B, int Hq, int Hkv, int Lmax, int D, double scale,
                          float *out)
{
    int g = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int n = count[(size_t)b * Hq + h];
            const int *ix = idx + ((size_t)b * Hq + h) * cap;
            const uint16_t *qv = q + ((size_t)b * Hq + h) * D;
            int kvh = h / g;
            double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            double *o = (double *)malloc(sizeof(double) * (size_t)D);
            double m = -INFINITY;
            for (int i = 0; i < n; ++i) {
                const uint16_t *kr = kc + (((size_t)b * Hkv + kvh) * Lmax + ix[i]) * D;
                double acc = 0.0;
                for (int c = 0; c < D; ++c)
                    acc += bf16_value(qv[c]) * bf16_value(kr[c]);
                z[i] = acc * scale;
                if (z[i] > m)
                    m = z[i];
            }
            double l = 0.0;
            for (int c = 0; c < D; ++c)
                o[c] = 0.0;
            for (int i = 0; i < n; ++i) {
                double p = exp(z[i] - m);
                const uint16_t *vr = vc + (((size_t)b * Hkv + kvh) * Lmax + ix[i]) * D;
                l += p;
                for (int c = 0; c < D; ++c)
                    o[c] += p * bf16_value(vr[c]);
            }
            float *dst = out + ((size_t)b * Hq + h) * D;
            for (int c = 0; c < D; ++c)
                dst[c] = n > 0 ? (float)(o[c] / l) : 0.0f;
            free(z);
            free(o);
        }
}
