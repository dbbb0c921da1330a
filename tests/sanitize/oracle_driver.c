/*
 * Driver for the fp64 oracle (oracle/m3_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: runs m3o_scan and m3o_decode_step over small
 * shapes (empty and one-token sequences, dstate 2, ranks 1-4, one and several
 * threads, with and without a state record) on deterministic pseudo-random
 * inputs, and checks the properties any correct run has: status codes,
 * finite outputs, the bad-size rejections, and that a one-token scan equals
 * one decode step on the same record.  Exit status 0 means every check held
 * and the sanitizers found nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int m3o_scan(int64_t Bt, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
             const double *x, const double *Bm, const double *Cm,
             const double *dt, const double *A, const double *theta,
             const double *lam, const double *h0, const double *Bprev0,
             const double *xprev0, double *y, double *h_out,
             double *Bprev_out, double *xprev_out, int nthreads);
int m3o_decode_step(int64_t Bt, int64_t H, int64_t P, int64_t N, int64_t R,
                    const double *x, const double *Bm, const double *Cm,
                    const double *dt, const double *A, const double *theta,
                    const double *lam, double *h, double *Bprev, double *xprev,
                    double *y);

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static double uniform(void)   /* xorshift64*, in [-1, 1) */
{
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
/* exactly n doubles from the heap (n may be 0: a one-element block that is never read) */
static double *fill(int64_t n, double lo, double hi)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
    return p;
}
static int all_finite(const double *p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int failures = 0;
#define CHECK(c, ...)                                        \
    do {                                                     \
        if (!(c)) {                                          \
            ++failures;                                      \
            fprintf(stderr, "check failed: " __VA_ARGS__);   \
            fprintf(stderr, "\n");                           \
        }                                                    \
    } while (0)

static void scan_case(int64_t Bt, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
                      int with_state, int threads)
{
    const int64_t tok = Bt * L * H, bh = Bt * H;
    double *x = fill(tok * R * P, -1, 1), *Bm = fill(tok * R * N, -1, 1), *Cm = fill(tok * R * N, -1, 1);
    /* the C entry point takes the decay rate per token, [Bt, L, H] */
    double *dt = fill(tok, 0.01, 1.0), *A = fill(tok, -2.0, -0.1), *th = fill(tok * (N / 2), -3, 3);
    double *lam = fill(tok, 0.0, 1.0);
    double *h0 = with_state ? fill(bh * N * P, -1, 1) : NULL;
    double *b0 = with_state ? fill(bh * R * N, -1, 1) : NULL;
    double *x0 = with_state ? fill(bh * R * P, -1, 1) : NULL;
    double *y = fill(tok * R * P, 0, 0), *h = fill(bh * N * P, 0, 0);
    double *bo = fill(bh * R * N, 0, 0), *xo = fill(bh * R * P, 0, 0);
    const int st = m3o_scan(Bt, L, H, P, N, R, x, Bm, Cm, dt, A, th, lam, h0, b0, x0, y, h, bo, xo,
                            threads);
    CHECK(st == 0, "scan B%lld L%lld H%lld P%lld N%lld R%lld: status %d", (long long)Bt,
          (long long)L, (long long)H, (long long)P, (long long)N, (long long)R, st);
    CHECK(all_finite(y, tok * R * P) && all_finite(h, bh * N * P), "scan outputs not finite");
    if (L >= 1 && with_state && Bt * H > 0) {
        /* the first token as one decode step on the input record */
        double *hd = fill(bh * N * P, 0, 0), *bd = fill(bh * R * N, 0, 0), *xd = fill(bh * R * P, 0, 0);
        double *y1 = fill(tok * R * P, 0, 0), *h1 = fill(bh * N * P, 0, 0);
        double *bo1 = fill(bh * R * N, 0, 0), *xo1 = fill(bh * R * P, 0, 0);
        memcpy(hd, h0, sizeof(double) * bh * N * P);
        memcpy(bd, b0, sizeof(double) * bh * R * N);
        memcpy(xd, x0, sizeof(double) * bh * R * P);
        /* token 0 of each (b, h): gather it into [Bt, H, ...] step arrays */
        double *sx = fill(bh * R * P, 0, 0), *sb = fill(bh * R * N, 0, 0), *sc = fill(bh * R * N, 0, 0);
        double *sdt = fill(bh, 0, 0), *sA = fill(bh, 0, 0), *sth = fill(bh * (N / 2), 0, 0);
        double *sl = fill(bh, 0, 0), *sy = fill(bh * R * P, 0, 0);
        for (int64_t b = 0; b < Bt; ++b)
            for (int64_t hh = 0; hh < H; ++hh) {
                const int64_t u = b * H + hh, t0 = (b * L) * H + hh;
                memcpy(sx + u * R * P, x + t0 * R * P, sizeof(double) * R * P);
                memcpy(sb + u * R * N, Bm + t0 * R * N, sizeof(double) * R * N);
                memcpy(sc + u * R * N, Cm + t0 * R * N, sizeof(double) * R * N);
                memcpy(sth + u * (N / 2), th + t0 * (N / 2), sizeof(double) * (N / 2));
                sdt[u] = dt[t0];
                sl[u] = lam[t0];
                sA[u] = A[t0];
            }
        CHECK(m3o_decode_step(Bt, H, P, N, R, sx, sb, sc, sdt, sA, sth, sl, hd, bd, xd, sy) == 0,
              "decode status");
        /* a one-token scan on the same record */
        double *x1 = fill(bh * R * P, 0, 0), *b1 = fill(bh * R * N, 0, 0), *c1 = fill(bh * R * N, 0, 0);
        memcpy(x1, sx, sizeof(double) * bh * R * P);
        memcpy(b1, sb, sizeof(double) * bh * R * N);
        memcpy(c1, sc, sizeof(double) * bh * R * N);
        CHECK(m3o_scan(Bt, 1, H, P, N, R, x1, b1, c1, sdt, sA, sth, sl, h0, b0, x0, y1, h1, bo1, xo1,
                       threads) == 0, "one-token scan status");
        CHECK(memcmp(sy, y1, sizeof(double) * bh * R * P) == 0, "decode y != one-token scan y");
        CHECK(memcmp(hd, h1, sizeof(double) * bh * N * P) == 0, "decode h != one-token scan h");
        CHECK(memcmp(bd, bo1, sizeof(double) * bh * R * N) == 0, "decode B_prev != scan record");
        free(hd); free(bd); free(xd); free(y1); free(h1); free(bo1); free(xo1);
        free(sx); free(sb); free(sc); free(sdt); free(sA); free(sth); free(sl); free(sy);
        free(x1); free(b1); free(c1);
    }
    free(x); free(Bm); free(Cm); free(dt); free(A); free(th); free(lam);
    free(h0); free(b0); free(x0); free(y); free(h); free(bo); free(xo);
}

int main(void)
{
    const int64_t shapes[][6] = {
        /* Bt, L, H, P, N, R */
        {1, 0, 1, 4, 2, 1},  {1, 1, 1, 4, 2, 1},  {2, 3, 2, 5, 4, 2},  {1, 17, 3, 16, 16, 1},
        {2, 65, 2, 8, 8, 4}, {0, 9, 2, 4, 4, 1},  {3, 40, 1, 3, 6, 3}, {1, 33, 4, 16, 32, 2},
    };
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        for (int ws = 0; ws < 2; ++ws)
            for (int th = 1; th <= 3; th += 2)
                scan_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4],
                          shapes[i][5], ws, th);
    /* bad sizes are rejected before any access */
    CHECK(m3o_scan(1, 4, 1, 4, 3, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                   NULL, NULL, NULL, NULL, 1) == -1, "odd dstate accepted");
    CHECK(m3o_scan(-1, 4, 1, 4, 4, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                   NULL, NULL, NULL, NULL, 1) == -1, "negative batch accepted");
    CHECK(m3o_decode_step(1, 1, 0, 4, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                          NULL, NULL) == -1, "zero headdim accepted");
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
