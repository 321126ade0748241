/*
 * attn_oracle.c -- the f64 CPU oracle for softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file: only the test suite, the package's smoke check and the bench's
 * CPU-baseline leg do. It shares no code, header or constant with the HIP
 * library; the two meet only at the bf16 bit patterns of the seeded inputs.
 *
 * What it computes is the plain definition of the operation, written out
 * naively in double precision (the tang paper judges every kernel against a
 * "pure f64" interpreter, §4 "Precision is a schedule" and §6
 * "Verification"):
 *
 *   for every batch b, query head h and query row i
 *     g    = h / (Hq / Hkv)                      grouped-query head map (§2.1
 *                                                "Views": heads as two dims)
 *     J_i  = { j in [0, Sk) : (!causal || j <= i + Sk - Sq)
 *                              && (window < 0 || j >= i + Sk - Sq - window) }
 *     s_j  = scale * sum_t Q[b,h,i,t] * K[b,g,j,t]          (pass 1)
 *     s_j <- softcap * tanh(s_j / softcap)          (soft cap, softcap > 0)
 *     s_j <- s_j - slope_h * |i + Sk - Sq - j|      (ALiBi, slopes given)
 *     m    = max_{j in J_i} s_j
 *     l    = sum_{j in J_i} exp(s_j - m)                     (pass 2)
 *     O    = sum_{j in J_i} exp(s_j - m) * V[b,g,j,:] / l
 *     LSE  = m + ln(l)
 *     if J_i is empty: O = 0 and LSE = -inf
 *
 * The paper's §2.3 "Rewrites" states that the online-softmax reduction the
 * fast kernels use replaces exactly this max and these two exponential sums,
 * and §6 lists its equality with two-pass softmax as a proved theorem; so the
 * two-pass form is the definition the fast path must reproduce up to
 * rounding. Masked keys are excluded from J_i rather than biased, which is
 * the guarded-read reading of §2.1 (an out-of-range read yields the
 * reduction's identity). LSE is the natural log of the sum of exponentials of
 * the scaled scores, the quantity the flash backward of §3 reads back.
 *
 * Inputs are the bf16 bit patterns the GPU reads; each is widened exactly
 * (bits << 16 gives the float32 pattern, then float -> double). The scale is
 * the float32 value handed to the GPU, widened to double.
 *
 * The window term is the sliding-window variant (no window: window < 0), the
 * two score lines the soft-cap and ALiBi variants (§7.3's variant table). A
 * change of the score or the mask leaves the monoid alone (§2.3 "Rewrites"),
 * so the definition is the same two passes over modified scores or a smaller
 * key set.
 *
 * Decode (one query row per stream and head, keys [0, len_b) of a cache of
 * capacity S_cap) is the same definition with J = [0, len_b).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC attn_oracle.c -lm. No fast-math: the
 * sums run in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Score modifiers of one row: none when softcap == 0 and slope == 0. */
typedef struct {
    double softcap;  /* > 0: soft cap */
    double slope;    /* ALiBi slope of the row's query head */
    int64_t dist0;   /* i + Sk - Sq - (key index of the first key passed) */
} score_mod;

static const score_mod no_mod = {0.0, 0.0, 0};

/*
 * Two-pass softmax attention of one query row over keys 0..nkeys-1 of one
 * (b, kv-head) slice. k and v point at that slice's first key row; rows are
 * d elements apart. s is caller scratch of nkeys doubles. Writes o[0..d-1]
 * and *lse.
 */
static void attend_row(const uint16_t *qrow, const uint16_t *k,
                       const uint16_t *v, int64_t nkeys, int d, double scale,
                       score_mod mod, double *s, double *o, double *lse)
{
    int t;
    int64_t j;

    for (t = 0; t < d; ++t)
        o[t] = 0.0;
    if (nkeys <= 0) {
        *lse = -INFINITY;
        return;
    }

    /* pass 1: scaled scores and their maximum */
    double m = -INFINITY;
    for (j = 0; j < nkeys; ++j) {
        const uint16_t *krow = k + j * (int64_t)d;
        double dot = 0.0;
        for (t = 0; t < d; ++t)
            dot += widen_bf16(qrow[t]) * widen_bf16(krow[t]);
        s[j] = scale * dot;
        if (mod.softcap > 0.0)
            s[j] = mod.softcap * tanh(s[j] / mod.softcap);
        if (mod.slope != 0.0)
            s[j] -= mod.slope * (double)llabs(mod.dist0 - j);
        if (s[j] > m)
            m = s[j];
    }

    /* pass 2: exponential weights, their sum, the weighted values */
    double l = 0.0;
    for (j = 0; j < nkeys; ++j) {
        const uint16_t *vrow = v + j * (int64_t)d;
        double w = exp(s[j] - m);
        l += w;
        for (t = 0; t < d; ++t)
            o[t] += w * widen_bf16(vrow[t]);
    }
    for (t = 0; t < d; ++t)
        o[t] /= l;
    *lse = m + log(l);
}

/* End of the keys visible to query row i: J_i ends at n (exclusive). */
static int64_t visible_keys(int64_t i, int64_t Sq, int64_t Sk, int causal)
{
    if (!causal)
        return Sk;
    int64_t n = i + (Sk - Sq) + 1;    /* keys j <= i + Sk - Sq */
    if (n < 0)
        n = 0;
    if (n > Sk)
        n = Sk;
    return n;
}

static int bad_shape(int B, int Hq, int Hkv, int d)
{
    return B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0;
}

/* Start of the keys visible to query row i under a window (0 without). */
static int64_t first_visible_key(int64_t i, int64_t Sq, int64_t Sk, int window)
{
    if (window < 0)
        return 0;
    int64_t lo = i + (Sk - Sq) - window;  /* keys j >= i + Sk - Sq - window */
    return lo < 0 ? 0 : lo;
}

/*
 * Prefill oracle. q: [B,Hq,Sq,d], k and v: [B,Hkv,Sk,d] bf16 bits.
 * rows: flat row ids r = (b*Hq + h)*Sq + i to evaluate, or NULL for all
 * B*Hq*Sq rows in order. window: the sliding window (< 0: none). Writes
 * o[nrows*d] and lse[nrows] (row order of `rows`). Returns 0, or -1 on a bad
 * argument.
 */
int oracle_attn_fwd_ext(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
                        int window, float softcap, const float *alibi, float scale,
                        const int64_t *rows, int64_t nrows, double *o, double *lse,
                        int nthreads)
{
    if (bad_shape(B, Hq, Hkv, d) || Sq < 0 || Sk < 0 || !(softcap >= 0.f))
        return -1;
    const int64_t total = (int64_t)B * Hq * Sq;
    if (rows == NULL)
        nrows = total;
    const int G = Hq / Hkv;
    const double sc = (double)scale;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (Sk > 0 ? (size_t)Sk : 1));
        if (s == NULL) {
#pragma omp atomic write
            err = 1;
        } else {
            int64_t n;
#pragma omp for schedule(dynamic, 16)
            for (n = 0; n < nrows; ++n) {
                int64_t r = rows ? rows[n] : n;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    err = 1;
                    continue;
                }
                int64_t i = r % Sq;
                int64_t bh = r / Sq;
                int64_t h = bh % Hq;
                int64_t b = bh / Hq;
                int64_t g = h / G;
                const uint16_t *qrow = q + r * (int64_t)d;
                const uint16_t *kh = k + (b * Hkv + g) * (int64_t)Sk * d;
                const uint16_t *vh = v + (b * Hkv + g) * (int64_t)Sk * d;
                const int64_t lo = first_visible_key(i, Sq, Sk, window);
                const int64_t hi = visible_keys(i, Sq, Sk, causal);
                score_mod mod = no_mod;
                mod.softcap = (double)softcap;
                mod.slope = alibi ? (double)alibi[h] : 0.0;
                mod.dist0 = i + (Sk - Sq) - lo;
                attend_row(qrow, kh + lo * d, vh + lo * d, hi - lo, d, sc, mod,
                           s, o + n * (int64_t)d, lse + n);
            }
            free(s);
        }
    }
    return err ? -1 : 0;
}

/* Prefill oracle with a window and no score modifier. */
int oracle_attn_fwd_window(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
                           int window, float scale, const int64_t *rows, int64_t nrows,
                           double *o, double *lse, int nthreads)
{
    return oracle_attn_fwd_ext(q, k, v, B, Hq, Hkv, Sq, Sk, d, causal, window, 0.f, NULL,
                               scale, rows, nrows, o, lse, nthreads);
}

/* Prefill oracle without a window. */
int oracle_attn_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
                    float scale, const int64_t *rows, int64_t nrows,
                    double *o, double *lse, int nthreads)
{
    return oracle_attn_fwd_window(q, k, v, B, Hq, Hkv, Sq, Sk, d, causal, -1, scale,
                                  rows, nrows, o, lse, nthreads);
}

/*
 * Decode oracle. q: [B,Hq,d]; kc, vc: [B,Hkv,S_cap,d]; lens: [B], each in
 * [0, S_cap]. Writes o[B*Hq*d], lse[B*Hq]. Returns 0 or -1.
 */
int oracle_attn_decode(const uint16_t *q, const uint16_t *kc,
                       const uint16_t *vc, const int32_t *lens, int B, int Hq,
                       int Hkv, int S_cap, int d, float scale, double *o,
                       double *lse, int nthreads)
{
    if (bad_shape(B, Hq, Hkv, d) || S_cap < 0)
        return -1;
    for (int b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] > S_cap)
            return -1;
    const int G = Hq / Hkv;
    const double sc = (double)scale;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (S_cap > 0 ? (size_t)S_cap : 1));
        if (s == NULL) {
#pragma omp atomic write
            err = 1;
        } else {
            int64_t n;
#pragma omp for schedule(dynamic, 4)
            for (n = 0; n < (int64_t)B * Hq; ++n) {
                int64_t h = n % Hq;
                int64_t b = n / Hq;
                int64_t g = h / G;
                const uint16_t *kh = kc + (b * Hkv + g) * (int64_t)S_cap * d;
                const uint16_t *vh = vc + (b * Hkv + g) * (int64_t)S_cap * d;
                attend_row(q + n * (int64_t)d, kh, vh, lens[b], d, sc, no_mod, s,
                           o + n * (int64_t)d, lse + n);
            }
            free(s);
        }
    }
    return err ? -1 : 0;
}

/*
 * The probability row of one query: p_j = exp(s_j - m) / l for j in J_i, and
 * 0 for masked keys. Writes p[Sk]. Returns 0 or -1. Used by the tests that pin
 * the oracle (rows of P sum to one and lie in [0, 1]).
 */
int oracle_attn_probs(const uint16_t *q, const uint16_t *k, int B, int Hq,
                      int Hkv, int Sq, int Sk, int d, int causal, float scale,
                      int64_t row, double *p)
{
    if (bad_shape(B, Hq, Hkv, d) || Sq <= 0 || Sk < 0)
        return -1;
    if (row < 0 || row >= (int64_t)B * Hq * Sq)
        return -1;
    const int G = Hq / Hkv;
    int64_t i = row % Sq, bh = row / Sq, h = bh % Hq, b = bh / Hq, g = h / G;
    const uint16_t *qrow = q + row * (int64_t)d;
    const uint16_t *kh = k + (b * Hkv + g) * (int64_t)Sk * d;
    int64_t n = visible_keys(i, Sq, Sk, causal), j;
    double m = -INFINITY, l = 0.0;
    for (j = 0; j < Sk; ++j)
        p[j] = 0.0;
    for (j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int t = 0; t < d; ++t)
            dot += widen_bf16(qrow[t]) * widen_bf16(kh[j * (int64_t)d + t]);
        p[j] = (double)scale * dot;
        if (p[j] > m)
            m = p[j];
    }
    for (j = 0; j < n; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (j = 0; j < n; ++j)
        p[j] /= l;
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
