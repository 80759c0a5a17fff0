/*
 * Calls every entry point of the CPU oracle (oracle/fa_oracle.c) on small
 * random inputs in every mode -- causal or not, key lengths including 0 and
 * N, block masks with ragged last blocks, sampled rows at the edges, decode
 * with empty caches, merges with empty parts -- and on rejected arguments.
 * Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitize.py: any out-of-bounds access, use of
 * uninitialised heap memory through a bad index, leak or undefined
 * arithmetic in the oracle stops it with an error.  Prints "ok" at the end.
 * Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int fa_oracle_fwd(const double *, const double *, const double *, double *, double *, int, int,
                  int, int, int, double, const int32_t *, const uint8_t *, int);
int fa_oracle_fwd_rows(const double *, const double *, const double *, double *, double *, int,
                       int, int, int, int, double, const int32_t *, const uint8_t *, int,
                       const int64_t *, int64_t);
int fa_oracle_bwd(const double *, const double *, const double *, const double *, double *,
                  double *, double *, double *, int, int, int, int, int, double, const int32_t *,
                  const uint8_t *, int);
int fa_oracle_bwd_sample(const double *, const double *, const double *, const double *, int, int,
                         int, double, int, const uint8_t *, int, const int64_t *, int64_t,
                         double *, const int64_t *, int64_t, double *, double *);
int fa_oracle_decode(const double *, const double *, const double *, double *, double *, int, int,
                     int, int, int, int, double, const int32_t *);
int fa_oracle_merge(const double *, const double *, int, int64_t, int, double *, double *);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *fill(size_t n)
{
    double *p = malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i)
        p[i] = urand();
    return p;
}
static int fails = 0;
static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s returned %d, expected %d\n", what, got, want);
        ++fails;
    }
}

static void dense_case(int B, int H, int N, int d, int causal, int padded, int mb)
{
    const size_t n = (size_t)B * H * N * d, r = (size_t)B * H * N;
    double *q = fill(n), *k = fill(n), *v = fill(n), *g = fill(n);
    double *o = malloc(sizeof(double) * n), *l = malloc(sizeof(double) * r);
    double *dq = malloc(sizeof(double) * n), *dk = malloc(sizeof(double) * n);
    double *dv = malloc(sizeof(double) * n), *D = malloc(sizeof(double) * r);
    int32_t *lens = NULL;
    if (padded) {
        lens = malloc(sizeof(int32_t) * B);
        for (int b = 0; b < B; ++b)
            lens[b] = b == 0 ? 0 : (b == 1 ? N : 1 + (int)((urand() + 1.0) * 0.5 * (N - 1)));
    }
    uint8_t *mask = NULL;
    int nb = 0;
    if (mb) {
        nb = (N + mb - 1) / mb;
        mask = malloc((size_t)nb * nb);
        for (int i = 0; i < nb * nb; ++i)
            mask[i] = urand() > 0.0;
        mask[0] = 0;                       /* an empty first row block */
    }
    const double scale = 1.0 / sqrt((double)d);
    expect(fa_oracle_fwd(q, k, v, o, l, B, H, N, d, causal, scale, lens, mask, mb), 0, "fwd");
    int64_t rows[4] = {0, N - 1, (int64_t)r - 1, (int64_t)(r / 2)};
    double *orow = malloc(sizeof(double) * 4 * d), *lrow = malloc(sizeof(double) * 4);
    expect(fa_oracle_fwd_rows(q, k, v, orow, lrow, B, H, N, d, causal, scale, lens, mask, mb, rows,
                              4), 0, "fwd_rows");
    free(orow);
    free(lrow);
    expect(fa_oracle_bwd(q, k, v, g, dq, dk, dv, D, B, H, N, d, causal, scale, lens, mask, mb), 0,
           "bwd");
    expect(fa_oracle_bwd(q, k, v, g, dq, dk, dv, NULL, B, H, N, d, causal, scale, lens, mask, mb), 0,
           "bwd without D");
    int64_t qr[3] = {0, N - 1, N / 2}, kr[3] = {N - 1, 0, N / 3};
    double *sq = malloc(sizeof(double) * 3 * d), *sk = malloc(sizeof(double) * 3 * d);
    double *sv = malloc(sizeof(double) * 3 * d);
    expect(fa_oracle_bwd_sample(q, k, v, g, N, d, causal, scale, padded ? lens[B - 1] : N, mask, mb,
                                qr, 3, sq, kr, 3, sk, sv), 0, "bwd_sample");
    free(q); free(k); free(v); free(g); free(o); free(l); free(dq); free(dk); free(dv); free(D);
    free(lens); free(mask); free(sq); free(sk); free(sv);
}

static void decode_case(int B, int H, int Nq, int Nk, int d, int causal)
{
    const size_t nq = (size_t)B * H * Nq * d, nk = (size_t)B * H * Nk * d;
    double *q = fill(nq), *k = fill(nk), *v = fill(nk);
    double *o = malloc(sizeof(double) * nq), *l = malloc(sizeof(double) * B * H * Nq);
    int32_t *lens = malloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; ++b)
        lens[b] = b == 0 ? 0 : (b == 1 ? Nk : (int)((urand() + 1.0) * 0.5 * Nk));
    expect(fa_oracle_decode(q, k, v, o, l, B, H, Nq, Nk, d, causal, 0.3, lens), 0, "decode");
    expect(fa_oracle_decode(q, k, v, o, l, B, H, Nq, Nk, d, causal, 0.3, NULL), 0, "decode full");
    free(q); free(k); free(v); free(o); free(l); free(lens);
}

static void merge_case(int S, int64_t R, int d)
{
    double *op = fill((size_t)S * R * d), *lp = fill((size_t)S * R);
    for (int64_t r = 0; r < R; ++r)
        lp[r] = -INFINITY;                 /* part 0 empty everywhere */
    for (int s = 0; s < S; ++s)
        lp[(size_t)s * R + R - 1] = -INFINITY;   /* last row empty in every part */
    double *o = malloc(sizeof(double) * R * d), *l = malloc(sizeof(double) * R);
    expect(fa_oracle_merge(op, lp, S, R, d, o, l), 0, "merge");
    free(op); free(lp); free(o); free(l);
}

int main(void)
{
    const int shapes[][4] = {{2, 2, 37, 8}, {3, 1, 1, 4}, {1, 2, 64, 16}, {3, 2, 50, 6}};
    for (int s = 0; s < 4; ++s)
        for (int causal = 0; causal < 2; ++causal)
            for (int padded = 0; padded < 2; ++padded)
                for (int mb = 0; mb <= 16; mb += 16) {
                    const int *x = shapes[s];
                    if (padded && x[0] < 3)
                        continue;      /* lengths 0, N and random need three batches */
                    dense_case(x[0], x[1], x[2], x[3], causal, padded, mb);
                }
    for (int causal = 0; causal < 2; ++causal) {
        decode_case(3, 2, 1, 50, 8, causal);
        decode_case(3, 1, 3, 7, 4, causal);
        decode_case(4, 1, 5, 3, 4, causal);   /* more queries than keys */
    }
    merge_case(3, 5, 4);
    merge_case(1, 1, 1);
    /* rejected arguments return an error without touching memory */
    double z = 0.0;
    int64_t bad = -1;
    expect(fa_oracle_fwd(&z, &z, &z, &z, &z, 0, 1, 1, 1, 0, 1.0, NULL, NULL, 0), 1, "fwd B=0");
    expect(fa_oracle_fwd_rows(&z, &z, &z, &z, &z, 1, 1, 1, 1, 0, 1.0, NULL, NULL, 0, &bad, 1), 1,
           "fwd_rows bad row");
    expect(fa_oracle_bwd_sample(&z, &z, &z, &z, 1, 1, 0, 1.0, 1, NULL, 0, &bad, 1, &z, &bad, 1, &z,
                                &z), 1, "bwd_sample bad row");
    expect(fa_oracle_decode(&z, &z, &z, &z, &z, 1, 1, 0, 1, 1, 0, 1.0, NULL), 1, "decode Nq=0");
    expect(fa_oracle_merge(&z, &z, 0, 1, 1, &z, &z), 1, "merge S=0");
    if (fails)
        return 1;
    printf("ok\n");
    return 0;
}
