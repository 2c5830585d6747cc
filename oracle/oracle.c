/*
 * oracle.c -- the fp64 CPU oracle for exact scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file or the library built from it; only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark do.  It shares no code, header, helper
 * or constant with the HIP library.
 *
 * What it computes is the plain definition, written out with no blocking,
 * fusion or reordering:
 *
 *   s_ij  = scale * sum_c q_ic k_jc                       (scores)
 *   a_ij  = exp(s_ij - m_i) / sum_{j visible} exp(s_ij - m_i),  m_i = max_j s_ij
 *   o_i   = sum_{j visible} a_ij v_j
 *   lse_i = m_i + ln(sum_{j visible} exp(s_ij - m_i))     (natural log)
 *
 * Pages followed (cited by title and section):
 *   [R]  "Transformer 架构的数学与计算深度解析：注意力机制的详尽研究报告"
 *        (menggq.pages.dev): sec. 2.2 (scores as dot products q_i.k_j),
 *        sec. 2.3 (division by sqrt(d_k)), sec. 2.4 (row softmax, rows sum to
 *        one, output A V as a convex combination of value rows), sec. 4.1
 *        (causal mask: -inf on the future, zero weight after the softmax),
 *        sec. 6.3 (online softmax recurrence).
 *   [IO] "从注意力到 IO 感知执行" (auturnal.com review, v10): sec. 8 and its
 *        equations (1)-(2): running max m, denominator l, un-normalised
 *        weighted sum u, rescaled by exp(m - m'), output u'/l'.  Sec. 8 also
 *        states that subtracting the max changes only the representation.
 *   [N]  "Transformer 笔记：注意力机制为什么会变成系统问题" (imreese.github.io):
 *        the KV-cache section: a decode step's query reads the cached K/V of
 *        all earlier tokens.
 *   [E]  the pwwt.cn engineering blog on Transformer algorithm evolution,
 *        sec. 2.3: grouped-query attention, groups of query heads share one
 *        K/V head.
 *
 * Readings where the pages are silent (each is listed in the design doc):
 *   - causal alignment for Nq != Nk is bottom-right: query row i sits at
 *     absolute position i + (Nk - Nq), so it sees keys j <= i + (Nk - Nq);
 *   - GQA groups are contiguous: KV head of query head h is h / (Hq / Hkv);
 *   - a row with no visible key (decode with seq_len 0) has o = 0 and
 *     lse = -inf;
 *   - the scale multiplies q.k before masking and the softmax.
 *
 * Layouts: every tensor is contiguous, row-major, fp64:
 *   q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], o [B,Hq,Nq,d], lse [B,Hq,Nq],
 *   weights [B,Hq,Nq,Nk].  Decode: q [B,Hq,d], caches [B,Hkv,Lmax,d],
 *   seq_lens int32 [B], o [B,Hq,d], lse [B,Hq].
 *
 * Every entry point returns 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of keys query row i may see.  [R] sec. 4.1 defines the square case:
 * token t attends to positions 1..t.  With 0-based indices and bottom-right
 * alignment this is keys 0..i+(Nk-Nq). */
static long visible_keys(long i, long Nq, long Nk, int causal)
{
    if (!causal)
        return Nk;
    long last = i + (Nk - Nq); /* last visible key index */
    if (last < 0)
        return 0;
    if (last >= Nk)
        return Nk;
    return last + 1;
}

/* One output row by the direct definition.  qrow: d values; K, V: nvis rows of
 * d values (row stride d); s: scratch of nvis doubles; w (optional) receives the
 * nvis weights a_ij. */
static void direct_row(const double *qrow, const double *K, const double *V,
                       long nvis, long d, double scale, double *s,
                       double *orow, double *lse_out, double *w)
{
    long j, c;
    if (nvis == 0) {
        for (c = 0; c < d; ++c)
            orow[c] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    /* [R] sec. 2.2-2.3: s_j = scale * q . k_j */
    for (j = 0; j < nvis; ++j) {
        double acc = 0.0;
        for (c = 0; c < d; ++c)
            acc += qrow[c] * K[j * d + c];
        s[j] = scale * acc;
    }
    /* [R] sec. 2.4, with the max subtracted as [IO] sec. 8 allows. */
    double m = s[0];
    for (j = 1; j < nvis; ++j)
        if (s[j] > m)
            m = s[j];
    double l = 0.0;
    for (j = 0; j < nvis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (j = 0; j < nvis; ++j)
        s[j] /= l; /* s now holds the weights a_j */
    if (w)
        memcpy(w, s, (size_t)nvis * sizeof(double));
    /* [R] sec. 2.4: o = sum_j a_j v_j */
    for (c = 0; c < d; ++c)
        orow[c] = 0.0;
    for (j = 0; j < nvis; ++j) {
        double a = s[j];
        for (c = 0; c < d; ++c)
            orow[c] += a * V[j * d + c];
    }
    *lse_out = m + log(l);
}

/* One output row by the blockwise recurrence of [IO] sec. 8, eqs. (1)-(2)
 * (the same recurrence as [R] sec. 6.3), with key blocks of size beta:
 *   m' = max(m, max_j s_j)
 *   l' = exp(m - m') l + sum_j exp(s_j - m')
 *   u' = exp(m - m') u + sum_j exp(s_j - m') v_j
 * starting from m = -inf, l = 0, u = 0, and o = u'/l' after the last block. */
static void blockwise_row(const double *qrow, const double *K, const double *V,
                          long nvis, long d, double scale, long beta,
                          double *s, double *u, double *orow, double *lse_out)
{
    long j0, j, c;
    double m = -INFINITY, l = 0.0;
    for (c = 0; c < d; ++c)
        u[c] = 0.0;
    for (j0 = 0; j0 < nvis; j0 += beta) {
        long j1 = j0 + beta < nvis ? j0 + beta : nvis;
        double mblk = -INFINITY;
        for (j = j0; j < j1; ++j) {
            double acc = 0.0;
            for (c = 0; c < d; ++c)
                acc += qrow[c] * K[j * d + c];
            s[j - j0] = scale * acc;
            if (s[j - j0] > mblk)
                mblk = s[j - j0];
        }
        double mnew = m > mblk ? m : mblk;
        double alpha = exp(m - mnew); /* exp(-inf) = 0 on the first block */
        l *= alpha;
        for (c = 0; c < d; ++c)
            u[c] *= alpha;
        for (j = j0; j < j1; ++j) {
            double p = exp(s[j - j0] - mnew);
            l += p;
            for (c = 0; c < d; ++c)
                u[c] += p * V[j * d + c];
        }
        m = mnew;
    }
    if (nvis == 0) {
        for (c = 0; c < d; ++c)
            orow[c] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    for (c = 0; c < d; ++c)
        orow[c] = u[c] / l;
    *lse_out = m + log(l);
}

static int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || d < 1)
        return -1;
    if (Hq % Hkv != 0)
        return -1;
    return 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}


/* One decode step per sequence against a paged KV cache ("Transformer 笔记：
 * 注意力机制为什么会变成系统问题", the FlashAttention / PagedAttention section,
 * and the pwwt.cn blog, sec. 3.3: the cache is cut into fixed-size blocks
 * placed anywhere in a pool).  Pool layout kp/vp [num_blocks, Hkv, bs, d];
 * logical row j of sequence b lives in physical block
 * block_table[b * max_blocks + j / bs], row j % bs.  seq_lens[b] is clamped
 * to [0, max_blocks * bs] and table entries to [0, num_blocks - 1]
 * (num_blocks == 0: every sequence is empty).  The rows of each (b, KV head)
 * are gathered into a contiguous buffer and attended exactly as in
 * oracle_decode. */
int oracle_decode_paged(const double *q, const double *kp, const double *vp,
                        const int32_t *block_table, const int32_t *seq_lens,
                        double *o, double *lse, int B, int Hq, int Hkv,
                        int num_blocks, int bs, int max_blocks, int d,
                        double scale, int nthreads)
{
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || num_blocks < 0 || bs < 1 ||
        max_blocks < 0 || d < 1)
        return -1;
    set_threads(nthreads);
    const long G = Hq / Hkv;
    const long Lmax = num_blocks > 0 ? (long)max_blocks * bs : 0;
    const long rows = (long)B * Hq;
    int bad = 0;
#pragma omp parallel
    {
        const size_t n = (size_t)(Lmax > 0 ? Lmax : 1);
        double *s = (double *)malloc(sizeof(double) * n);
        double *K = (double *)malloc(sizeof(double) * n * (size_t)d);
        double *V = (double *)malloc(sizeof(double) * n * (size_t)d);
        if (!s || !K || !V) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < rows; ++r) {
            if (!s || !K || !V)
                continue;
            long b = r / Hq, h = r % Hq, hk = h / G;
            long L = seq_lens[b];
            if (L < 0)
                L = 0;
            if (L > Lmax)
                L = Lmax;
            for (long j = 0; j < L; ++j) {
                long blk = block_table[b * (long)max_blocks + j / bs];
                if (blk < 0)
                    blk = 0;
                if (blk > num_blocks - 1)
                    blk = num_blocks - 1;
                const long src = ((blk * Hkv + hk) * (long)bs + j % bs) * d;
                memcpy(K + j * d, kp + src, sizeof(double) * (size_t)d);
                memcpy(V + j * d, vp + src, sizeof(double) * (size_t)d);
            }
            direct_row(q + r * d, K, V, L, d, scale, s, o + r * d, lse + r, NULL);
        }
        free(s);
        free(K);
        free(V);
    }
    return bad ? -1 : 0;
}
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Full attention over every (b, h, i).  weights may be NULL; when given it has
 * B*Hq*Nq*Nk entries and receives a_ij (zero where j is masked). */
int oracle_attn(const double *q, const double *k, const double *v, double *o,
                double *lse, double *weights, int B, int Hq, int Hkv, int Nq,
                int Nk, int d, double scale, int causal, int nthreads)
{
    if (check_shape(B, Hq, Hkv, Nq, Nk, d))
        return -1;
    set_threads(nthreads);
    const long G = Hq / Hkv;
    const long rows = (long)B * Hq * Nq;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < rows; ++r) {
            if (!s)
                continue;
            long i = r % Nq;
            long h = (r / Nq) % Hq;
            long b = r / ((long)Nq * Hq);
            long hk = h / G; /* contiguous groups, [E] sec. 2.3 */
            const double *qrow = q + r * d;
            const double *K = k + ((b * Hkv + hk) * (long)Nk) * d;
            const double *V = v + ((b * Hkv + hk) * (long)Nk) * d;
            long nvis = visible_keys(i, Nq, Nk, causal);
            double *w = NULL;
            if (weights) {
                w = weights + r * (long)Nk;
                memset(w, 0, sizeof(double) * (size_t)Nk);
            }
            direct_row(qrow, K, V, nvis, d, scale, s, o + r * d, lse + r, w);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* The same definition for a list of rows only: rows holds n triples
 * (b, h, i); o receives n*d values and lse n values, in list order. */
int oracle_attn_rows(const double *q, const double *k, const double *v,
                     const int32_t *rows, long n, double *o, double *lse, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, double scale,
                     int causal, int nthreads)
{
    if (check_shape(B, Hq, Hkv, Nq, Nk, d))
        return -1;
    for (long t = 0; t < n; ++t) {
        if (rows[3 * t] < 0 || rows[3 * t] >= B || rows[3 * t + 1] < 0 ||
            rows[3 * t + 1] >= Hq || rows[3 * t + 2] < 0 || rows[3 * t + 2] >= Nq)
            return -1;
    }
    set_threads(nthreads);
    const long G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long t = 0; t < n; ++t) {
            if (!s)
                continue;
            long b = rows[3 * t], h = rows[3 * t + 1], i = rows[3 * t + 2];
            long hk = h / G;
            const double *qrow = q + (((b * Hq + h) * (long)Nq) + i) * d;
            const double *K = k + ((b * Hkv + hk) * (long)Nk) * d;
            const double *V = v + ((b * Hkv + hk) * (long)Nk) * d;
            long nvis = visible_keys(i, Nq, Nk, causal);
            direct_row(qrow, K, V, nvis, d, scale, s, o + t * d, lse + t, NULL);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* Full attention by the blockwise recurrence with block size beta >= 1. */
int oracle_blockwise(const double *q, const double *k, const double *v,
                     double *o, double *lse, int B, int Hq, int Hkv, int Nq,
                     int Nk, int d, double scale, int causal, int beta,
                     int nthreads)
{
    if (check_shape(B, Hq, Hkv, Nq, Nk, d) || beta < 1)
        return -1;
    set_threads(nthreads);
    const long G = Hq / Hkv;
    const long rows = (long)B * Hq * Nq;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)beta);
        double *u = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !u) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < rows; ++r) {
            if (!s || !u)
                continue;
            long i = r % Nq;
            long h = (r / Nq) % Hq;
            long b = r / ((long)Nq * Hq);
            long hk = h / G;
            const double *K = k + ((b * Hkv + hk) * (long)Nk) * d;
            const double *V = v + ((b * Hkv + hk) * (long)Nk) * d;
            long nvis = visible_keys(i, Nq, Nk, causal);
            blockwise_row(q + r * d, K, V, nvis, d, scale, beta, s, u, o + r * d,
                          lse + r);
        }
        free(s);
        free(u);
    }
    return bad ? -1 : 0;
}

/* One decode step per sequence: the single query of (b, h) attends to the
 * first seq_lens[b] cached rows of KV head h / (Hq/Hkv), per [N]'s KV-cache
 * section.  seq_lens[b] is clamped to [0, Lmax]. */
int oracle_decode(const double *q, const double *kc, const double *vc,
                  const int32_t *seq_lens, double *o, double *lse, int B, int Hq,
                  int Hkv, int Lmax, int d, double scale, int nthreads)
{
    if (check_shape(B, Hq, Hkv, 1, Lmax, d))
        return -1;
    set_threads(nthreads);
    const long G = Hq / Hkv;
    const long rows = (long)B * Hq;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Lmax > 0 ? Lmax : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < rows; ++r) {
            if (!s)
                continue;
            long b = r / Hq, h = r % Hq, hk = h / G;
            long L = seq_lens[b];
            if (L < 0)
                L = 0;
            if (L > Lmax)
                L = Lmax;
            const double *K = kc + ((b * Hkv + hk) * (long)Lmax) * d;
            const double *V = vc + ((b * Hkv + hk) * (long)Lmax) * d;
            direct_row(q + r * d, K, V, L, d, scale, s, o + r * d, lse + r, NULL);
        }
        free(s);
    }
    return bad ? -1 : 0;
}
