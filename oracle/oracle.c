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
 * and, for the backward pass, the chain-rule gradients dq, dk, dv of that
 * definition for an upstream gradient do of o (see oracle_attn_bwd).
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
 * Readings where the pages are silent:
 *   - causal alignment for Nq != Nk is bottom-right: query row i sits at
 *     absolute position i + (Nk - Nq), so it sees keys j <= i + (Nk - Nq);
 *   - GQA groups are contiguous: KV head of query head h is h / (Hq / Hkv);
 *   - a row with no visible key (decode with seq_len 0) has o = 0 and
 *     lse = -inf;
 *   - the scale multiplies q.k before masking and the softmax.
 *
 * Layouts: every tensor is contiguous, row-major, fp64:
 *   q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], o [B,Hq,Nq,d], lse [B,Hq,Nq],
 *   weights [B,Hq,Nq,Nk]; do/dq as q, dk/dv as k.  Decode: q [B,Hq,d], caches [B,Hkv,Lmax,d],
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

/* ---------------------------------------------------------------------------
 * Backward pass (gradients of the forward definition above).
 *
 * The pages state that training needs the gradients of attention ([R]
 * sec. 3.3: the standard implementation keeps the N x N matrix for the
 * backward pass), that FlashAttention recomputes instead of storing it
 * ("Transformer 深度进阶" [M], the FlashAttention section: recomputation adds
 * FLOPs but cuts memory traffic), and that an exact tiled kernel is checked by
 * comparing outputs AND gradients with a higher-precision reference ([IO],
 * the evaluation protocol).  They print no gradient formula.  The oracle
 * therefore takes the derivative of the forward definition by the chain rule,
 * for an upstream gradient dO of the output:
 *
 *   dv_j  = sum_i a_ij do_i                       (o_i = sum_j a_ij v_j)
 *   dp_ij = do_i . v_j                            (dL/da_ij)
 *   ds_ij = a_ij (dp_ij - sum_k a_ik dp_ik)       (softmax Jacobian)
 *   dq_i  = scale * sum_j ds_ij k_j               (s_ij = scale q_i.k_j)
 *   dk_j  = scale * sum_i ds_ij q_i
 *
 * with masked pairs contributing nothing, and for GQA the sum over every
 * query head of the group into the shared K/V head's dk, dv.  A finite-
 * difference test of the forward pins these formulas.
 * ------------------------------------------------------------------------ */

/* Gradient contributions of one query row.  qrow, dorow: d values; K, V: the
 * nvis visible rows; a, dp: scratch of nvis doubles; dqrow receives dq_i;
 * dK, dV (row stride d) accumulate this row's share of dk_j, dv_j. */
static void bwd_row(const double *qrow, const double *dorow, const double *K,
                    const double *V, long nvis, long d, double scale, double *a,
                    double *dp, double *orow_scratch, double *dqrow, double *dK,
                    double *dV)
{
    long j, c;
    double lse;
    for (c = 0; c < d; ++c)
        dqrow[c] = 0.0;
    if (nvis == 0)
        return;
    direct_row(qrow, K, V, nvis, d, scale, dp, orow_scratch, &lse, a); /* a_ij */
    double D = 0.0;
    for (j = 0; j < nvis; ++j) {
        double acc = 0.0;
        for (c = 0; c < d; ++c)
            acc += dorow[c] * V[j * d + c];
        dp[j] = acc;
        D += a[j] * acc;
    }
    for (j = 0; j < nvis; ++j) {
        double ds = a[j] * (dp[j] - D);
        for (c = 0; c < d; ++c) {
            dqrow[c] += scale * ds * K[j * d + c];
            dK[j * d + c] += scale * ds * qrow[c];
            dV[j * d + c] += a[j] * dorow[c];
        }
    }
}

/* Full backward: dq [B,Hq,Nq,d], dk/dv [B,Hkv,Nk,d] (layouts as the forward),
 * from q, k, v and the upstream gradient do_ [B,Hq,Nq,d].  One (b, KV head)
 * per task, so each task owns its dk/dv rows. */
int oracle_attn_bwd(const double *q, const double *k, const double *v,
                    const double *do_, double *dq, double *dk, double *dv,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, double scale,
                    int causal, int nthreads)
{
    if (check_shape(B, Hq, Hkv, Nq, Nk, d))
        return -1;
    set_threads(nthreads);
    const long G = Hq / Hkv;
    const long groups = (long)B * Hkv;
    int bad = 0;
#pragma omp parallel
    {
        const size_t n = (size_t)(Nk > 0 ? Nk : 1);
        double *a = (double *)malloc(sizeof(double) * n);
        double *dp = (double *)malloc(sizeof(double) * n);
        double *orow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!a || !dp || !orow) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long t = 0; t < groups; ++t) {
            if (!a || !dp || !orow)
                continue;
            long b = t / Hkv, hk = t % Hkv;
            const long kv0 = ((b * Hkv + hk) * (long)Nk) * d;
            double *dK = dk + kv0, *dV = dv + kv0;
            memset(dK, 0, sizeof(double) * (size_t)Nk * d);
            memset(dV, 0, sizeof(double) * (size_t)Nk * d);
            for (long h = hk * G; h < (hk + 1) * G; ++h) { /* [E] sec. 2.3 */
                for (long i = 0; i < Nq; ++i) {
                    const long r = ((b * Hq + h) * (long)Nq + i) * d;
                    bwd_row(q + r, do_ + r, k + kv0, v + kv0,
                            visible_keys(i, Nq, Nk, causal), d, scale, a, dp,
                            orow, dq + r, dK, dV);
                }
            }
        }
        free(a);
        free(dp);
        free(orow);
    }
    return bad ? -1 : 0;
}

/* Selected gradient rows of the same definition, for sizes where the full
 * backward is too slow: dq for the nq query rows qrows (triples b, h, i) and
 * dk, dv for the nk key rows krows (triples b, hk, j).
 *
 * A key row's gradient needs, for every query row i of its group that sees
 * it, the weight a_ij and D_i = sum_k a_ik dp_ik; with lse_i the log of the
 * row's denominator, a_ij = exp(s_ij - lse_i) ([R] sec. 2.4 written with the
 * log-sum-exp).  Both statistics come from the direct definition of each such
 * row, then the key row sums its terms over i in index order. */
int oracle_attn_bwd_rows(const double *q, const double *k, const double *v,
                         const double *do_, const int32_t *qrows, long nq,
                         const int32_t *krows, long nk, double *dq_out,
                         double *dk_out, double *dv_out, int B, int Hq, int Hkv,
                         int Nq, int Nk, int d, double scale, int causal,
                         int nthreads)
{
    if (check_shape(B, Hq, Hkv, Nq, Nk, d))
        return -1;
    for (long t = 0; t < nq; ++t)
        if (qrows[3 * t] < 0 || qrows[3 * t] >= B || qrows[3 * t + 1] < 0 ||
            qrows[3 * t + 1] >= Hq || qrows[3 * t + 2] < 0 || qrows[3 * t + 2] >= Nq)
            return -1;
    for (long t = 0; t < nk; ++t)
        if (krows[3 * t] < 0 || krows[3 * t] >= B || krows[3 * t + 1] < 0 ||
            krows[3 * t + 1] >= Hkv || krows[3 * t + 2] < 0 || krows[3 * t + 2] >= Nk)
            return -1;
    set_threads(nthreads);
    const long G = Hq / Hkv;
    int bad = 0;

    /* dq rows: each is the dq of bwd_row, with the dk/dv shares discarded */
#pragma omp parallel
    {
        const size_t n = (size_t)(Nk > 0 ? Nk : 1);
        double *a = (double *)malloc(sizeof(double) * n);
        double *dp = (double *)malloc(sizeof(double) * n);
        double *orow = (double *)malloc(sizeof(double) * (size_t)d);
        double *sink = (double *)calloc(n * (size_t)d * 2, sizeof(double));
        if (!a || !dp || !orow || !sink) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long t = 0; t < nq; ++t) {
            if (!a || !dp || !orow || !sink)
                continue;
            long b = qrows[3 * t], h = qrows[3 * t + 1], i = qrows[3 * t + 2];
            long hk = h / G;
            const long r = ((b * Hq + h) * (long)Nq + i) * d;
            const long kv0 = ((b * Hkv + hk) * (long)Nk) * d;
            bwd_row(q + r, do_ + r, k + kv0, v + kv0, visible_keys(i, Nq, Nk, causal),
                    d, scale, a, dp, orow, dq_out + t * d, sink, sink + n * (size_t)d);
        }
        free(a);
        free(dp);
        free(orow);
        free(sink);
    }
    if (bad || nk == 0)
        return bad ? -1 : 0;

    /* statistics (lse_i, D_i) of every row of every group that a key row names */
    char *need = (char *)calloc((size_t)B * Hkv, 1);
    double *lse = (double *)malloc(sizeof(double) * (size_t)B * Hq * (Nq > 0 ? Nq : 1));
    double *Dst = (double *)malloc(sizeof(double) * (size_t)B * Hq * (Nq > 0 ? Nq : 1));
    if (!need || !lse || !Dst) {
        free(need);
        free(lse);
        free(Dst);
        return -1;
    }
    for (long t = 0; t < nk; ++t)
        need[krows[3 * t] * (long)Hkv + krows[3 * t + 1]] = 1;
    const long rows = (long)B * Hq * Nq;
#pragma omp parallel
    {
        const size_t n = (size_t)(Nk > 0 ? Nk : 1);
        double *a = (double *)malloc(sizeof(double) * n);
        double *sc = (double *)malloc(sizeof(double) * n);
        double *orow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!a || !sc || !orow) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < rows; ++r) {
            if (!a || !sc || !orow)
                continue;
            long i = r % Nq, h = (r / Nq) % Hq, b = r / ((long)Nq * Hq), hk = h / G;
            if (!need[b * Hkv + hk])
                continue;
            const long kv0 = ((b * Hkv + hk) * (long)Nk) * d;
            long nvis = visible_keys(i, Nq, Nk, causal);
            direct_row(q + r * d, k + kv0, v + kv0, nvis, d, scale, sc, orow, lse + r, a);
            double D = 0.0;
            for (long j = 0; j < nvis; ++j) {
                double acc = 0.0;
                for (long c = 0; c < d; ++c)
                    acc += do_[r * d + c] * v[kv0 + j * d + c];
                D += a[j] * acc;
            }
            Dst[r] = D;
        }
        free(a);
        free(sc);
        free(orow);
    }
    /* dk, dv rows */
#pragma omp parallel for schedule(dynamic, 1)
    for (long t = 0; t < nk; ++t) {
        if (bad)
            continue;
        long b = krows[3 * t], hk = krows[3 * t + 1], j = krows[3 * t + 2];
        const double *kj = k + (((b * Hkv + hk) * (long)Nk) + j) * d;
        const double *vj = v + (((b * Hkv + hk) * (long)Nk) + j) * d;
        double *dkr = dk_out + t * d, *dvr = dv_out + t * d;
        for (long c = 0; c < d; ++c) {
            dkr[c] = 0.0;
            dvr[c] = 0.0;
        }
        for (long h = hk * G; h < (hk + 1) * G; ++h) {
            for (long i = 0; i < Nq; ++i) {
                if (j >= visible_keys(i, Nq, Nk, causal))
                    continue;
                const long r = (b * Hq + h) * (long)Nq + i;
                const double *qi = q + r * d, *doi = do_ + r * d;
                double s = 0.0, dpv = 0.0;
                for (long c = 0; c < d; ++c) {
                    s += qi[c] * kj[c];
                    dpv += doi[c] * vj[c];
                }
                const double aij = exp(scale * s - lse[r]);
                const double ds = aij * (dpv - Dst[r]);
                for (long c = 0; c < d; ++c) {
                    dkr[c] += scale * ds * qi[c];
                    dvr[c] += aij * doi[c];
                }
            }
        }
    }
    free(need);
    free(lse);
    free(Dst);
    return bad ? -1 : 0;
}
