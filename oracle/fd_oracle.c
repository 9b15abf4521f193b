/*
 * fd_oracle.c -- plain, slow, fp64 CPU oracle for split-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; it includes only the C standard library.
 *
 * Sources (pages; sections as printed on them):
 *   [P1] "FlashDecoding 数学推导" (my-webpage-adu.pages.dev, 2026-07-15)
 *   [P2] "adv04: Flash-Decoding（长序列 Decode 切分 + FlashInfer 简介）"
 *        (mini-vllm-tutorial.vercel.app)
 *   [P3] "FlashDecoding 数学推导：传统 m/l/o 方法与 LSE 方法"
 *        (my-webpage-adu.pages.dev, 2026-07-16)
 *
 * What is computed, and in which precision:
 *   Every input element is decoded exactly to double (fp32, IEEE binary16
 *   and bfloat16 all embed exactly in binary64) and every sum, exp and log
 *   is taken in double.  Attention is the plain definition: the scores of the
 *   one query row against all keys, a max-shifted softmax over the whole row,
 *   and the softmax-weighted sum of the value rows ([P1] §2.1.1, §2.3.1;
 *   [P3] §2.1.1).  Because the split method reaches exactly this result
 *   ([P1] §2.6, [P3] §2.2.3 and §2.3.6), the full-row definition is the
 *   oracle for the whole decode step; the per-split partials and the merges
 *   are written out separately so that each GPU stage can be checked alone.
 *
 * Layouts (row-major, innermost last):
 *   q      [batch, heads_q, d]
 *   k, v   [batch, max_kv_len, heads_kv, d]
 *   o      [rows, d] (double), lse [rows] (double)
 *   o_part [batch, heads_q, num_splits, d], lse_part [batch, heads_q, num_splits]
 * Query head hq reads key/value head hq / (heads_q / heads_kv): consecutive
 * query heads form one group per key/value head.  The pages only name
 * grouped-query attention; this contiguous grouping is the reading taken.
 *
 * Parallelism: (batch, query head) pairs are independent; OpenMP spreads the
 * pairs over threads when the library is built with -fopenmp.  Within a pair
 * the arithmetic is sequential in token order, exactly as written below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

/* ------------------------------------------------------------------------ */
/* Element decoding, written from the IEEE-754 / bfloat16 bit layouts.       */
/* ------------------------------------------------------------------------ */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 7) & 0xff;
    int frac = h & 0x7f;
    double mag;
    if (expo == 0xff)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, 1 - 127 - 7); /* subnormal: 0.frac x 2^-126 */
    else
        mag = ldexp((double)(frac | 0x80), expo - 127 - 7); /* 1.frac x 2^(e-127) */
    return sign ? -mag : mag;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0x1f)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, 1 - 15 - 10); /* subnormal: 0.frac x 2^-14 */
    else
        mag = ldexp((double)(frac | 0x400), expo - 15 - 10);
    return sign ? -mag : mag;
}

/* Decode element `idx` of an array stored in `dtype`. */
static double elem(const void *base, int dtype, size_t idx)
{
    if (dtype == OR_F32) {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char *)base + idx * 2, 2);
    return dtype == OR_F16 ? oracle_f16_to_f64(h) : oracle_bf16_to_f64(h);
}

/* Bulk decode (used by the tests to compare the decoders with numpy). */
void oracle_decode(int dtype, const void *src, size_t n, double *dst)
{
    for (size_t i = 0; i < n; ++i)
        dst[i] = elem(src, dtype, i);
}

/* ------------------------------------------------------------------------ */
/* Softmax on a plain vector.                                               */
/* ------------------------------------------------------------------------ */

/* Max-shifted softmax: p_i = exp(x_i - m) / sum_j exp(x_j - m), m = max x
 * ([P1] §2.3.1).  n >= 1. */
void oracle_softmax(const double *x, int n, double *p)
{
    double m = x[0];
    for (int i = 1; i < n; ++i)
        if (x[i] > m)
            m = x[i];
    double sum = 0.0;
    for (int i = 0; i < n; ++i)
        sum += exp(x[i] - m);
    for (int i = 0; i < n; ++i)
        p[i] = exp(x[i] - m) / sum;
}

/* Online softmax recurrence ([P1] §2.3.2): m_1 = x_1, d_1 = 1, then
 *   m_j = max(m_{j-1}, x_j),  d_j = d_{j-1} exp(m_{j-1} - m_j) + exp(x_j - m_j).
 * Writes the running (m_j, d_j) for every j into m_trace / d_trace (length n). */
void oracle_online_softmax(const double *x, int n, double *m_trace, double *d_trace)
{
    double m = x[0], d = 1.0;
    m_trace[0] = m;
    d_trace[0] = d;
    for (int j = 1; j < n; ++j) {
        double m_new = x[j] > m ? x[j] : m;
        d = d * exp(m - m_new) + exp(x[j] - m_new);
        m = m_new;
        m_trace[j] = m;
        d_trace[j] = d;
    }
}

/* ------------------------------------------------------------------------ */
/* One (sequence, query head): scores and the direct tile statistics.       */
/* ------------------------------------------------------------------------ */

/* s_j = scale * sum_k q[k] K_j[k] for tokens j in [t0, t1) of sequence b,
 * key/value head kvh ([P1] §2.2; [P3] §2.1.1). */
static void scores(int dtype, const void *q, const void *k, int b, int hq, int kvh,
                   int heads_q, int heads_kv, int max_kv_len, int d, double scale,
                   int t0, int t1, double *s)
{
    size_t q_off = ((size_t)b * heads_q + hq) * d;
    for (int j = t0; j < t1; ++j) {
        size_t k_off = (((size_t)b * max_kv_len + j) * heads_kv + kvh) * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += elem(q, dtype, q_off + c) * elem(k, dtype, k_off + c);
        s[j - t0] = scale * dot;
    }
}

/* Direct per-tile statistics over tokens [t0, t1), t1 > t0 ([P1] §2.4.1,
 * direct form; [P3] §2.2.1 and §2.3.3):
 *   m = max_j s_j,  l = sum_j exp(s_j - m),
 *   o = sum_j exp(s_j - m) V_j / l.
 * `s` holds the t1 - t0 scores; o has d entries. */
static void tile_stats(int dtype, const void *v, int b, int kvh, int heads_kv, int max_kv_len,
                       int d, int t0, int t1, const double *s, double *m_out, double *l_out,
                       double *o)
{
    int n = t1 - t0;
    double m = s[0];
    for (int j = 1; j < n; ++j)
        if (s[j] > m)
            m = s[j];
    double l = 0.0;
    for (int c = 0; c < d; ++c)
        o[c] = 0.0;
    for (int j = 0; j < n; ++j) {
        double w = exp(s[j] - m);
        l += w;
        size_t v_off = (((size_t)b * max_kv_len + (t0 + j)) * heads_kv + kvh) * d;
        for (int c = 0; c < d; ++c)
            o[c] += w * elem(v, dtype, v_off + c);
    }
    for (int c = 0; c < d; ++c)
        o[c] /= l;
    *m_out = m;
    *l_out = l;
}

static int seq_len(const int32_t *kv_lens, int b, int max_kv_len)
{
    if (!kv_lens)
        return max_kv_len;
    int n = kv_lens[b];
    if (n < 0)
        n = 0;
    if (n > max_kv_len)
        n = max_kv_len;
    return n;
}

/* ------------------------------------------------------------------------ */
/* Full decode attention: the plain definition.                             */
/* ------------------------------------------------------------------------ */

/* For each requested (b, hq) pair:
 *   o   = softmax(q K^T * scale) V  over the sequence's kv_lens[b] tokens,
 *   lse = log sum_j exp(s_j) = m + log l   (natural log, scaled scores;
 *         [P3] §2.3.1 safe form).
 * An empty sequence gives o = 0 and lse = -inf (the identity of the merge,
 * [P3] §3.2.1 initial state).
 * rows: n_rows pairs (b, hq) as int32[2 * n_rows]; NULL means every pair in
 * (b, hq) order and n_rows is ignored.  kv_lens: NULL means all max_kv_len.
 * Returns 0, or -1 if a scratch allocation fails. */
int oracle_attention(int dtype, const void *q, const void *k, const void *v,
                     const int32_t *kv_lens, int batch, int heads_q, int heads_kv,
                     int max_kv_len, int d, double scale, int n_rows, const int32_t *rows,
                     double *o, double *lse)
{
    int group = heads_q / heads_kv;
    long total = rows ? n_rows : (long)batch * heads_q;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (max_kv_len > 0 ? max_kv_len : 1));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < total; ++r) {
            if (!s)
                continue;
            int b = rows ? rows[2 * r] : (int)(r / heads_q);
            int hq = rows ? rows[2 * r + 1] : (int)(r % heads_q);
            int kvh = hq / group;
            int n = seq_len(kv_lens, b, max_kv_len);
            double *orow = o + (size_t)r * d;
            if (n == 0) {
                for (int c = 0; c < d; ++c)
                    orow[c] = 0.0;
                lse[r] = -INFINITY;
                continue;
            }
            scores(dtype, q, k, b, hq, kvh, heads_q, heads_kv, max_kv_len, d, scale, 0, n, s);
            double m, l;
            tile_stats(dtype, v, b, kvh, heads_kv, max_kv_len, d, 0, n, s, &m, &l, orow);
            lse[r] = m + log(l);
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Per-split partials: the same direct formula restricted to each split.    */
/* ------------------------------------------------------------------------ */

/* Split i of sequence b covers tokens [i*L, min((i+1)*L, N_b)) ([P1] §2.5
 * step 2a; [P2] §4 chunking by ceil(seq / num_splits)).  For every split this
 * writes the LSE pair ([P3] §2.3.3):
 *   o_part = sum_j exp(s_j - m) V_j / l,   lse_part = S = m + log l,
 * and, when m_part / l_part are non-NULL, the triple's m and l ([P3] §2.2.1).
 * An empty split writes o = 0, S = -inf, m = -inf, l = 0. */
int oracle_split_partials(int dtype, const void *q, const void *k, const void *v,
                          const int32_t *kv_lens, int batch, int heads_q, int heads_kv,
                          int max_kv_len, int d, double scale, int num_splits, int split_len,
                          double *o_part, double *lse_part, double *m_part, double *l_part)
{
    int group = heads_q / heads_kv;
    long total = (long)batch * heads_q;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (split_len > 0 ? split_len : 1));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < total; ++r) {
            if (!s)
                continue;
            int b = (int)(r / heads_q), hq = (int)(r % heads_q), kvh = hq / group;
            int n = seq_len(kv_lens, b, max_kv_len);
            for (int i = 0; i < num_splits; ++i) {
                size_t slot = (size_t)r * num_splits + i;
                double *orow = o_part + slot * d;
                long t0 = (long)i * split_len;
                long t1 = t0 + split_len < n ? t0 + split_len : n;
                if (t0 >= t1) {
                    for (int c = 0; c < d; ++c)
                        orow[c] = 0.0;
                    lse_part[slot] = -INFINITY;
                    if (m_part)
                        m_part[slot] = -INFINITY;
                    if (l_part)
                        l_part[slot] = 0.0;
                    continue;
                }
                scores(dtype, q, k, b, hq, kvh, heads_q, heads_kv, max_kv_len, d, scale,
                       (int)t0, (int)t1, s);
                double m, l;
                tile_stats(dtype, v, b, kvh, heads_kv, max_kv_len, d, (int)t0, (int)t1, s, &m,
                           &l, orow);
                lse_part[slot] = m + log(l);
                if (m_part)
                    m_part[slot] = m;
                if (l_part)
                    l_part[slot] = l;
            }
        }
        free(s);
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Merges.                                                                   */
/* ------------------------------------------------------------------------ */

/* LSE merge of B partials per row ([P3] §2.3.4, stage 3 of §3.2.1):
 *   S_g = log sum_b exp(S_b)   (taken as S_max + log sum_b exp(S_b - S_max)),
 *   o   = sum_b exp(S_b - S_g) o_b.
 * Terms with S_b = -inf (empty splits) contribute nothing; a row whose every
 * S_b is -inf gives o = 0, S_g = -inf. */
void oracle_combine(const double *o_part, const double *lse_part, long rows, int num_splits,
                    int d, double *o, double *lse)
{
    for (long r = 0; r < rows; ++r) {
        const double *S = lse_part + (size_t)r * num_splits;
        const double *op = o_part + (size_t)r * num_splits * d;
        double *orow = o + (size_t)r * d;
        double smax = -INFINITY;
        for (int i = 0; i < num_splits; ++i)
            if (S[i] > smax)
                smax = S[i];
        for (int c = 0; c < d; ++c)
            orow[c] = 0.0;
        if (smax == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int i = 0; i < num_splits; ++i)
            if (S[i] != -INFINITY)
                sum += exp(S[i] - smax);
        double sg = smax + log(sum);
        for (int i = 0; i < num_splits; ++i) {
            if (S[i] == -INFINITY)
                continue;
            double w = exp(S[i] - sg);
            for (int c = 0; c < d; ++c)
                orow[c] += w * op[(size_t)i * d + c];
        }
        lse[r] = sg;
    }
}

/* The two-operand merge (o1, S1) (+) (o2, S2) in its stable form ([P3] §2.3.5
 * for the operator, §3.2.1 stage 2 for the stable evaluation):
 *   S = S_max + log(1 + exp(S_min - S_max)),
 *   o = o1 exp(S1 - S) + o2 exp(S2 - S).
 * (0, -inf) is the identity: merging with it returns the other operand. */
void oracle_merge2(const double *o1, double s1, const double *o2, double s2, int d, double *o,
                   double *s)
{
    if (s1 == -INFINITY && s2 == -INFINITY) {
        for (int c = 0; c < d; ++c)
            o[c] = 0.0;
        *s = -INFINITY;
        return;
    }
    double smax = s1 > s2 ? s1 : s2;
    double smin = s1 > s2 ? s2 : s1;
    double sm = smax + log1p(exp(smin - smax));
    double w1 = exp(s1 - sm), w2 = exp(s2 - sm);
    for (int c = 0; c < d; ++c)
        o[c] = o1[c] * w1 + o2[c] * w2;
    *s = sm;
}

/* The m/l/o merge of B triples per row ([P1] §2.4.2, stage 2 of §2.5;
 * [P3] §2.2.2):
 *   m_g = max_b m_b,  l_g = sum_b exp(m_b - m_g) l_b,
 *   o   = sum_b exp(m_b - m_g) l_b o_b / l_g.
 * Empty splits (m = -inf, l = 0) contribute nothing; a row with no tokens gives
 * o = 0, m_g = -inf, l_g = 0. */
void oracle_combine_mlo(const double *o_part, const double *m_part, const double *l_part,
                        long rows, int num_splits, int d, double *o, double *m_out,
                        double *l_out)
{
    for (long r = 0; r < rows; ++r) {
        const double *m = m_part + (size_t)r * num_splits;
        const double *l = l_part + (size_t)r * num_splits;
        const double *op = o_part + (size_t)r * num_splits * d;
        double *orow = o + (size_t)r * d;
        double mg = -INFINITY;
        for (int i = 0; i < num_splits; ++i)
            if (m[i] > mg)
                mg = m[i];
        for (int c = 0; c < d; ++c)
            orow[c] = 0.0;
        if (mg == -INFINITY) {
            m_out[r] = -INFINITY;
            l_out[r] = 0.0;
            continue;
        }
        double lg = 0.0;
        for (int i = 0; i < num_splits; ++i)
            if (m[i] != -INFINITY)
                lg += exp(m[i] - mg) * l[i];
        for (int i = 0; i < num_splits; ++i) {
            if (m[i] == -INFINITY)
                continue;
            double w = exp(m[i] - mg) * l[i];
            for (int c = 0; c < d; ++c)
                orow[c] += w * op[(size_t)i * d + c];
        }
        for (int c = 0; c < d; ++c)
            orow[c] /= lg;
        m_out[r] = mg;
        l_out[r] = lg;
    }
}

/* Incremental (online) statistics of one tile ([P1] §2.4.1, incremental
 * form): m_1 = s_1, l_1 = 1, o_1 = V_1, then for j >= 2
 *   m_j = max(m_{j-1}, s_j),
 *   l_j = l_{j-1} exp(m_{j-1} - m_j) + exp(s_j - m_j),
 *   o_j = (l_{j-1} exp(m_{j-1} - m_j) o_{j-1} + exp(s_j - m_j) V_j) / l_j.
 * Inputs are plain doubles: q[d], kmat[n][d], vmat[n][d]; scores use `scale`.
 * Writes the running m_j, l_j and o_j (o_trace[n][d]). */
void oracle_tile_incremental(const double *q, const double *kmat, const double *vmat, int n,
                             int d, double scale, double *m_trace, double *l_trace,
                             double *o_trace)
{
    double m = 0.0, l = 0.0;
    for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int c = 0; c < d; ++c)
            s += q[c] * kmat[(size_t)j * d + c];
        s *= scale;
        double *oj = o_trace + (size_t)j * d;
        const double *vj = vmat + (size_t)j * d;
        if (j == 0) {
            m = s;
            l = 1.0;
            for (int c = 0; c < d; ++c)
                oj[c] = vj[c];
        } else {
            const double *oprev = o_trace + (size_t)(j - 1) * d;
            double m_new = s > m ? s : m;
            double carry = l * exp(m - m_new);
            double w = exp(s - m_new);
            double l_new = carry + w;
            for (int c = 0; c < d; ++c)
                oj[c] = (carry * oprev[c] + w * vj[c]) / l_new;
            m = m_new;
            l = l_new;
        }
        m_trace[j] = m;
        l_trace[j] = l;
    }
}

/* Threads the OpenMP runtime would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
