/*
 * fa_oracle.c -- plain, slow, fp64 CPU oracle for exact scaled dot-product
 * attention and its gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file.  Its only users are the tests, the package's smoke check and
 * the CPU-baseline leg of the benchmark.  It shares no code, header or table
 * with the GPU library.
 *
 * What it computes (and why it is written this way)
 * -------------------------------------------------
 * The pages say the tiled method reaches exactly the result of ordinary
 * attention, only faster ("The Attention Matrix You Never Write Down", section
 * "The running-statistics trick"; "FlashAttention Explained", reference notes
 * 01 and 06).  So the oracle is that ordinary result written out, with no
 * tiling and no online softmax: the three moves of "01 · FlashAttention",
 * step 2 of 5 "Ordinary attention", and the definition
 * O = softmax(Q K^T / sqrt(d)) V of "FlashAttention: Mathematical Foundations,
 * IO-Aware Tiling, Online Softmax, and Recomputation Dynamics", section "The
 * GPU Memory Hierarchy and the Attention Memory Wall".  Softmax is the safe
 * form of that page's section "Online Softmax: The Mathematical Core" (subtract
 * the row maximum, sum the exponentials, divide).
 *
 * Each score row is materialised in full (O(N) doubles per thread).
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *  - causal: key j is allowed for query i iff j <= i;
 *  - key padding: key j is allowed iff j < kv_len[b]; every query row is
 *    still computed;
 *  - block mask: the mask "zeroes" a block by excluding its keys from the
 *    softmax (score minus infinity, probability 0), never by setting the
 *    score to 0 ("Attention" chapter of learn-kernels.com, paragraph on
 *    block-sparse FlashAttention);
 *  - the stored row statistic is one log-sum-exp LSE = m + ln(l) in natural
 *    log units of the scaled scores;
 *  - a row with no allowed key has O = 0, LSE = -inf and zero gradients;
 *  - the backward pass is the chain rule of the same definition with the loss
 *    L = sum(O * dO); the pages only name dQ, dK, dV ("FlashAttention:
 *    Mathematical Foundations ...", section "Backward Pass and Activation
 *    Recomputation").  D_i is formed as sum_j P_ij dP_ij, not as dO_i . O_i,
 *    so that it does not depend on any shortcut of the GPU path.
 *
 * Layout: every tensor is [B][H][N][d] (d innermost), LSE and D are
 * [B][H][N], kv_len is [B] (nullable), block_mask is [nb][nb] row-major with
 * nb = ceil(N / mask_block) (nullable), shared by every (b, h).
 *
 * Parity pins: see tests/test_oracle.py (brute force in 40-digit decimal,
 * closed forms, invariants, finite differences, a library autograd).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int fa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Is key j visible to query i of batch entry b? */
static int allowed(int i, int j, int causal, int kv_len,
                   const uint8_t *mask, int nb, int mask_block)
{
    if (causal && j > i)
        return 0;
    if (j >= kv_len)
        return 0;
    if (mask && !mask[(size_t)(i / mask_block) * nb + (size_t)(j / mask_block)])
        return 0;
    return 1;
}

static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t)
        s += a[t] * b[t];
    return s;
}

/*
 * One query row: fills p[0..N) with the softmax probabilities (0 for keys that
 * are not allowed) and returns the row's log-sum-exp (-inf when no key is
 * allowed, in which case p is all zero).
 */
static double softmax_row(const double *qi, const double *kh, int N, int d,
                          int i, int causal, int kv_len, const uint8_t *mask,
                          int nb, int mask_block, double scale,
                          double *s, unsigned char *ok, double *p)
{
    /* move 1: scores of the allowed keys */
    double m = -INFINITY;
    int any = 0;
    for (int j = 0; j < N; ++j) {
        ok[j] = (unsigned char)allowed(i, j, causal, kv_len, mask, nb, mask_block);
        if (ok[j]) {
            s[j] = scale * dot(qi, kh + (size_t)j * d, d);
            if (!any || s[j] > m)
                m = s[j];
            any = 1;
        }
    }
    if (!any) {
        memset(p, 0, sizeof(double) * (size_t)N);
        return -INFINITY;
    }
    /* move 2: safe softmax -- subtract the row maximum, sum, divide */
    double l = 0.0;
    for (int j = 0; j < N; ++j)
        if (ok[j])
            l += exp(s[j] - m);
    for (int j = 0; j < N; ++j)
        p[j] = ok[j] ? exp(s[j] - m) / l : 0.0;
    return m + log(l);
}

/* Forward over the rows listed in rows[] (indices into the B*H*N row space),
 * or over every row when rows == NULL.  o_out/lse_out are indexed like rows
 * (row r of the output is rows[r]) when rows is given, else [B][H][N]. */
static int fwd_impl(const double *q, const double *k, const double *v,
                    double *o, double *lse, int B, int H, int N, int d,
                    int causal, double scale, const int32_t *kv_lens,
                    const uint8_t *mask, int mask_block,
                    const int64_t *rows, int64_t nrows)
{
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return 1;
    if (mask && mask_block <= 0)
        return 1;
    const int nb = mask ? (N + mask_block - 1) / mask_block : 0;
    const int64_t total = rows ? nrows : (int64_t)B * H * N;
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *p = (double *)malloc(sizeof(double) * (size_t)N);
        unsigned char *ok = (unsigned char *)malloc((size_t)N);
        if (!s || !p || !ok) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < total; ++r) {
                const int64_t g = rows ? rows[r] : r; /* global row id */
                const int64_t bh = g / N;
                const int i = (int)(g % N);
                const int b = (int)(bh / H);
                const int kvl = kv_lens ? kv_lens[b] : N;
                const double *qi = q + (size_t)g * d;
                const double *kh = k + (size_t)bh * N * d;
                const double *vh = v + (size_t)bh * N * d;
                const double L = softmax_row(qi, kh, N, d, i, causal, kvl, mask,
                                             nb, mask_block, scale, s, ok, p);
                /* move 3: O_i = sum_j P_ij v_j */
                double *oi = o + (size_t)r * d;
                for (int t = 0; t < d; ++t)
                    oi[t] = 0.0;
                for (int j = 0; j < N; ++j)
                    if (p[j] != 0.0)
                        for (int t = 0; t < d; ++t)
                            oi[t] += p[j] * vh[(size_t)j * d + t];
                lse[r] = L;
            }
        }
        free(s);
        free(p);
        free(ok);
    }
    return err;
}

int fa_oracle_fwd(const double *q, const double *k, const double *v,
                  double *o, double *lse, int B, int H, int N, int d,
                  int causal, double scale, const int32_t *kv_lens,
                  const uint8_t *mask, int mask_block)
{
    return fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, kv_lens, mask,
                    mask_block, NULL, 0);
}

/* Forward for a sample of rows; rows[r] = (b*H + h)*N + i. */
int fa_oracle_fwd_rows(const double *q, const double *k, const double *v,
                       double *o, double *lse, int B, int H, int N, int d,
                       int causal, double scale, const int32_t *kv_lens,
                       const uint8_t *mask, int mask_block,
                       const int64_t *rows, int64_t nrows)
{
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)B * H * N)
            return 1;
    return fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, kv_lens, mask,
                    mask_block, rows, nrows);
}

/*
 * Backward, chain rule of the definition with L = sum(O * dO):
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i
 * Parallel over (b, h); rows of one head run in order so that dK and dV
 * accumulate without races.  D (nullable) receives D_i.
 */
int fa_oracle_bwd(const double *q, const double *k, const double *v,
                  const double *dout, double *dq, double *dk, double *dv,
                  double *dvec, int B, int H, int N, int d, int causal,
                  double scale, const int32_t *kv_lens, const uint8_t *mask,
                  int mask_block)
{
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
        return 1;
    if (mask && mask_block <= 0)
        return 1;
    const int nb = mask ? (N + mask_block - 1) / mask_block : 0;
    const size_t nd = (size_t)N * d;
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *p = (double *)malloc(sizeof(double) * (size_t)N);
        double *dp = (double *)malloc(sizeof(double) * (size_t)N);
        unsigned char *ok = (unsigned char *)malloc((size_t)N);
        if (!s || !p || !dp || !ok) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
                const int b = (int)(bh / H);
                const int kvl = kv_lens ? kv_lens[b] : N;
                const double *qh = q + (size_t)bh * nd;
                const double *kh = k + (size_t)bh * nd;
                const double *vh = v + (size_t)bh * nd;
                const double *doh = dout + (size_t)bh * nd;
                double *dqh = dq + (size_t)bh * nd;
                double *dkh = dk + (size_t)bh * nd;
                double *dvh = dv + (size_t)bh * nd;
                memset(dqh, 0, sizeof(double) * nd);
                memset(dkh, 0, sizeof(double) * nd);
                memset(dvh, 0, sizeof(double) * nd);
                for (int i = 0; i < N; ++i) {
                    const double *qi = qh + (size_t)i * d;
                    const double *doi = doh + (size_t)i * d;
                    softmax_row(qi, kh, N, d, i, causal, kvl, mask, nb,
                                mask_block, scale, s, ok, p);
                    double D = 0.0;
                    for (int j = 0; j < N; ++j) {
                        dp[j] = ok[j] ? dot(doi, vh + (size_t)j * d, d) : 0.0;
                        D += p[j] * dp[j];
                    }
                    if (dvec)
                        dvec[(size_t)bh * N + i] = D;
                    double *dqi = dqh + (size_t)i * d;
                    for (int j = 0; j < N; ++j) {
                        if (!ok[j])
                            continue;
                        const double ds = p[j] * (dp[j] - D);
                        const double *kj = kh + (size_t)j * d;
                        double *dkj = dkh + (size_t)j * d;
                        double *dvj = dvh + (size_t)j * d;
                        for (int t = 0; t < d; ++t) {
                            dqi[t] += scale * ds * kj[t];
                            dkj[t] += scale * ds * qi[t];
                            dvj[t] += p[j] * doi[t];
                        }
                    }
                }
            }
        }
        free(s);
        free(p);
        free(dp);
        free(ok);
    }
    return err;
}

/*
 * Backward for a sample of one head (b, h), for checks at sizes where the
 * full backward is too slow: dQ for the query rows qrows[0..nq) and dK, dV
 * for the key rows krows[0..nk).  dK_j and dV_j need P_ij for every query
 * row i, which needs every row's statistics; those come from the same
 * definition (row by row, no sharing with the GPU path).
 */
int fa_oracle_bwd_sample(const double *q, const double *k, const double *v,
                         const double *dout, int N, int d, int causal,
                         double scale, int kv_len, const uint8_t *mask,
                         int mask_block, const int64_t *qrows, int64_t nq,
                         double *dq_rows, const int64_t *krows, int64_t nk,
                         double *dk_rows, double *dv_rows)
{
    if (N <= 0 || d <= 0 || (mask && mask_block <= 0))
        return 1;
    for (int64_t r = 0; r < nq; ++r)
        if (qrows[r] < 0 || qrows[r] >= N)
            return 1;
    for (int64_t r = 0; r < nk; ++r)
        if (krows[r] < 0 || krows[r] >= N)
            return 1;
    const int nb = mask ? (N + mask_block - 1) / mask_block : 0;
    int err = 0;
    memset(dk_rows, 0, sizeof(double) * (size_t)nk * d);
    memset(dv_rows, 0, sizeof(double) * (size_t)nk * d);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *p = (double *)malloc(sizeof(double) * (size_t)N);
        double *dp = (double *)malloc(sizeof(double) * (size_t)N);
        unsigned char *ok = (unsigned char *)malloc((size_t)N);
        double *dk_loc = (double *)calloc((size_t)nk * d + 1, sizeof(double));
        double *dv_loc = (double *)calloc((size_t)nk * d + 1, sizeof(double));
        if (!s || !p || !dp || !ok || !dk_loc || !dv_loc) {
#pragma omp atomic write
            err = 2;
        } else {
            /* dQ rows */
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nq; ++r) {
                const int i = (int)qrows[r];
                const double *qi = q + (size_t)i * d;
                const double *doi = dout + (size_t)i * d;
                softmax_row(qi, k, N, d, i, causal, kv_len, mask, nb,
                            mask_block, scale, s, ok, p);
                double D = 0.0;
                for (int j = 0; j < N; ++j) {
                    dp[j] = ok[j] ? dot(doi, v + (size_t)j * d, d) : 0.0;
                    D += p[j] * dp[j];
                }
                double *dqi = dq_rows + (size_t)r * d;
                for (int t = 0; t < d; ++t)
                    dqi[t] = 0.0;
                for (int j = 0; j < N; ++j) {
                    if (!ok[j])
                        continue;
                    const double ds = p[j] * (dp[j] - D);
                    for (int t = 0; t < d; ++t)
                        dqi[t] += scale * ds * k[(size_t)j * d + t];
                }
            }
            /* dK, dV rows: every query row contributes */
            if (nk > 0) {
#pragma omp for schedule(dynamic, 8)
                for (int i = 0; i < N; ++i) {
                    const double *qi = q + (size_t)i * d;
                    const double *doi = dout + (size_t)i * d;
                    softmax_row(qi, k, N, d, i, causal, kv_len, mask, nb,
                                mask_block, scale, s, ok, p);
                    double D = 0.0;
                    for (int j = 0; j < N; ++j) {
                        dp[j] = ok[j] ? dot(doi, v + (size_t)j * d, d) : 0.0;
                        D += p[j] * dp[j];
                    }
                    for (int64_t r = 0; r < nk; ++r) {
                        const int j = (int)krows[r];
                        if (!ok[j])
                            continue;
                        const double ds = p[j] * (dp[j] - D);
                        for (int t = 0; t < d; ++t) {
                            dk_loc[(size_t)r * d + t] += scale * ds * qi[t];
                            dv_loc[(size_t)r * d + t] += p[j] * doi[t];
                        }
                    }
                }
#pragma omp critical
                {
                    for (size_t t = 0; t < (size_t)nk * d; ++t) {
                        dk_rows[t] += dk_loc[t];
                        dv_rows[t] += dv_loc[t];
                    }
                }
            }
        }
        free(s);
        free(p);
        free(dp);
        free(ok);
        free(dk_loc);
        free(dv_loc);
    }
    return err;
}

/*
 * Decode-shaped forward: Nq new query rows per (b, h) against a key/value
 * cache of Nk rows, of which the first kv_len[b] are filled (all Nk when
 * kv_lens is NULL).  The pages name this case -- the cache grows by one
 * token per step and each step is a small matmul ("Attention" chapter of
 * learn-kernels.com, paragraph on decoding) -- and the result is the same
 * definition as above with a rectangular score matrix.
 *
 * Reading where the pages are silent: the Nq queries are the newest Nq
 * positions of the sequence, so query t sits at position kv_len - Nq + t.
 * Without the causal flag every query sees keys j < kv_len; with it, query t
 * sees keys j <= kv_len - Nq + t (the square causal mask aligned at the
 * bottom right; for Nq = 1 both are the same).  A query that sees no key has
 * O = 0 and LSE = -inf.
 *
 * Layout: q and o are [B][H][Nq][d], k and v are [B][H][Nk][d], lse is
 * [B][H][Nq].
 */
int fa_oracle_decode(const double *q, const double *k, const double *v,
                     double *o, double *lse, int B, int H, int Nq, int Nk,
                     int d, int causal, double scale, const int32_t *kv_lens)
{
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
        return 1;
    const int64_t total = (int64_t)B * H * Nq;
    int err = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
        if (!s) {
#pragma omp atomic write
            err = 2;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < total; ++r) {
                const int64_t bh = r / Nq;
                const int t = (int)(r % Nq);
                const int b = (int)(bh / H);
                int len = kv_lens ? kv_lens[b] : Nk;
                if (len > Nk)
                    len = Nk;
                /* keys j < visible are allowed for this query */
                int visible = causal ? len - Nq + t + 1 : len;
                if (visible < 0)
                    visible = 0;
                const double *qi = q + (size_t)r * d;
                const double *kh = k + (size_t)bh * Nk * d;
                const double *vh = v + (size_t)bh * Nk * d;
                double *oi = o + (size_t)r * d;
                for (int e = 0; e < d; ++e)
                    oi[e] = 0.0;
                if (visible == 0) {
                    lse[r] = -INFINITY;
                    continue;
                }
                /* move 1: scores; move 2: safe softmax; move 3: O = P V */
                double m = -INFINITY;
                for (int j = 0; j < visible; ++j) {
                    s[j] = scale * dot(qi, kh + (size_t)j * d, d);
                    if (s[j] > m)
                        m = s[j];
                }
                double l = 0.0;
                for (int j = 0; j < visible; ++j)
                    l += exp(s[j] - m);
                for (int j = 0; j < visible; ++j) {
                    const double p = exp(s[j] - m) / l;
                    for (int e = 0; e < d; ++e)
                        oi[e] += p * vh[(size_t)j * d + e];
                }
                lse[r] = m + log(l);
            }
        }
        free(s);
    }
    return err;
}

/*
 * Combine S partial results of the same rows, each computed over a disjoint
 * part of the keys: o_parts is [S][R][d] (each part's own normalised output)
 * and lse_parts is [S][R] (each part's log-sum-exp, natural log, -inf for a
 * part with no key).  The parts are folded in order with the two-block
 * update of "FlashAttention: Mathematical Foundations, IO-Aware Tiling,
 * Online Softmax, and Recomputation Dynamics", section "Incremental Online
 * Updates", written in log-sum-exp form: with l = exp(LSE - m), the weight
 * that page gives the first block's output, l1 exp(m1 - m_new) / l_new,
 * equals exp(LSE1 - LSE_new), and likewise for the second block.
 * The result is O [R][d] and LSE [R]; rows where every part is empty get
 * O = 0 and LSE = -inf.
 */
int fa_oracle_merge(const double *o_parts, const double *lse_parts, int S,
                    int64_t R, int d, double *o, double *lse)
{
    if (S <= 0 || R < 0 || d <= 0)
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        double *oi = o + (size_t)r * d;
        double L = -INFINITY;   /* running log-sum-exp of the folded parts */
        for (int e = 0; e < d; ++e)
            oi[e] = 0.0;
        for (int s = 0; s < S; ++s) {
            const double Ls = lse_parts[(size_t)s * R + r];
            if (Ls == -INFINITY)
                continue;   /* an empty part contributes nothing */
            const double *os = o_parts + ((size_t)s * R + r) * d;
            if (L == -INFINITY) {
                for (int e = 0; e < d; ++e)
                    oi[e] = os[e];
                L = Ls;
                continue;
            }
            /* m_new = max(m1, m2); l_new = l1 e^(m1-m_new) + l2 e^(m2-m_new) */
            const double mx = L > Ls ? L : Ls;
            const double Lnew = mx + log(exp(L - mx) + exp(Ls - mx));
            const double w1 = exp(L - Lnew), w2 = exp(Ls - Lnew);
            for (int e = 0; e < d; ++e)
                oi[e] = w1 * oi[e] + w2 * os[e];
            L = Lnew;
        }
        lse[r] = L;
    }
    return 0;
}
