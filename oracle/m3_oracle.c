/*
 * m3_oracle.c -- fp64 CPU oracle for the Mamba-3 sequence mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP library is checked against.  It shares no code, header, table or helper
 * with the GPU path, and only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  Nothing in the product calls it.
 *
 * What it computes (per batch row b and head h, every step in double):
 *
 *   Mamba-3 summary on b-lab.team, section 1 "Exponential-Trapezoidal
 *   Discretization", the recurrence and its shorthand:
 *       h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1} + gamma_t B_t x_t
 *       alpha_t = exp(dt_t A),  beta_t = (1 - lam_t) dt_t exp(dt_t A),
 *       gamma_t = lam_t dt_t,   lam_t in [0, 1].
 *   Same page, section 2 "Complex-Valued State Space Model": the state
 *   transition of the complex SSM, written as a real SSM of size N, is
 *   exp(dt_t A) R_t with R_t block-diagonal in N/2 two-by-two rotations
 *   R(dt_t theta_t[i]),  R(phi) = [[cos phi, -sin phi], [sin phi, cos phi]],
 *   acting on adjacent state rows (2i, 2i+1).  The readout is y_t = C_t^T h_t.
 *   Same page, section 3 "MIMO": B_t is N x R, the input X_t is R x P, so the
 *   input term is the matrix product B_t X_t (a sum over the R ranks), and the
 *   readout C_t^T h_t gives one P-vector per rank.
 *
 * Readings taken where the pages leave a step open:
 *   - The rotation R_t multiplies the previous-endpoint term as well as
 *     h_{t-1}: the trapezoid's left endpoint is carried across the interval by
 *     the same flow exp(dt_t (A + i theta_t)) as the state (the complex SSM of
 *     section 2 discretised with the rule of section 1).  Without it the
 *     scheme is only first order at lam = 1/2.
 *   - beta_t uses the current step's lam_t and dt_t (as printed).
 *   - At the first step the previous endpoint B_0 X_0 is zero unless the caller
 *     supplies it in the state record (B_prev, x_prev).
 *   - The returned final state is h_L itself; the pending trapezoid term of a
 *     step L+1 is not folded in.  Instead (B_L, X_L) are returned so that a
 *     later scan or decode step can supply it.
 *
 * The decay rate is taken per token, A_t, as section 1 of the same page
 * writes it (exp(dt_t A_t)); a rate constant per head is the special case
 * A_t = A_h, which the Python wrapper passes broadcast.
 *
 * Layouts (row-major, contiguous, all double):
 *   x      [Bt, L, H, R, P]      Bm, Cm [Bt, L, H, R, N]
 *   dt,lam [Bt, L, H]            theta  [Bt, L, H, N/2]     A [Bt, L, H]
 *   h      [Bt, H, N, P]         Bprev  [Bt, H, R, N]       xprev [Bt, H, R, P]
 *   y      [Bt, L, H, R, P]
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t Bt, L, H, P, N, R;
    const double *x, *Bm, *Cm, *dt, *A, *theta, *lam;
    const double *h0, *Bprev0, *xprev0;   /* nullable: zero state, zero cache */
    double *y, *h_out, *Bprev_out, *xprev_out;   /* h_out etc. nullable */
    int64_t next_unit;                     /* work counter, guarded by mu */
    pthread_mutex_t mu;
    int status;
} scan_job;

/* U[n][p] = sum_r Bm[r][n] * X[r][p]  (the N x P product B_t X_t). */
static void input_term(const double *Bm, const double *X, int64_t N, int64_t P,
                       int64_t R, double *U)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t p = 0; p < P; ++p) {
            double s = 0.0;
            for (int64_t r = 0; r < R; ++r)
                s += Bm[r * N + n] * X[r * P + p];
            U[n * P + p] = s;
        }
}

/*
 * One step of the recurrence on a single (b, h) unit, in place:
 *   h <- alpha R h + beta R Uprev + gamma U ;  y = C^T h.
 * h and Uprev are N x P.  Uprev is the previous step's B X (the caller keeps
 * it); U is this step's B X.  Cm is R x N, y is R x P.
 */
static void step(double *h, const double *Uprev, const double *U,
                 const double *Cm, double dt, double A, const double *theta,
                 double lam, int64_t N, int64_t P, int64_t R, double *y)
{
    const double alpha = exp(dt * A);
    const double beta = (1.0 - lam) * dt * alpha;
    const double gamma = lam * dt;
    for (int64_t i = 0; i < N / 2; ++i) {
        const double phi = dt * theta[i];
        const double c = cos(phi), s = sin(phi);
        double *h0 = h + (2 * i) * P, *h1 = h + (2 * i + 1) * P;
        const double *u0 = Uprev + (2 * i) * P, *u1 = Uprev + (2 * i + 1) * P;
        const double *v0 = U + (2 * i) * P, *v1 = U + (2 * i + 1) * P;
        for (int64_t p = 0; p < P; ++p) {
            /* R(phi) applied to the pair (row 2i, row 2i+1) */
            const double rh0 = c * h0[p] - s * h1[p];
            const double rh1 = s * h0[p] + c * h1[p];
            const double ru0 = c * u0[p] - s * u1[p];
            const double ru1 = s * u0[p] + c * u1[p];
            h0[p] = alpha * rh0 + beta * ru0 + gamma * v0[p];
            h1[p] = alpha * rh1 + beta * ru1 + gamma * v1[p];
        }
    }
    for (int64_t r = 0; r < R; ++r)
        for (int64_t p = 0; p < P; ++p) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                s += Cm[r * N + n] * h[n * P + p];
            y[r * P + p] = s;
        }
}

static void scan_unit(const scan_job *j, int64_t b, int64_t hh, double *h,
                      double *Uprev, double *U)
{
    const int64_t L = j->L, H = j->H, P = j->P, N = j->N, R = j->R;
    const int64_t bh = b * H + hh;
    if (j->h0) memcpy(h, j->h0 + bh * N * P, sizeof(double) * N * P);
    else memset(h, 0, sizeof(double) * N * P);
    if (j->Bprev0 && j->xprev0)
        input_term(j->Bprev0 + bh * R * N, j->xprev0 + bh * R * P, N, P, R, Uprev);
    else memset(Uprev, 0, sizeof(double) * N * P);

    for (int64_t t = 0; t < L; ++t) {
        const int64_t bth = (b * L + t) * H + hh;
        const double *Bt = j->Bm + bth * R * N;
        const double *Xt = j->x + bth * R * P;
        input_term(Bt, Xt, N, P, R, U);
        step(h, Uprev, U, j->Cm + bth * R * N, j->dt[bth], j->A[bth],
             j->theta + bth * (N / 2), j->lam[bth], N, P, R, j->y + bth * R * P);
        double *tmp = Uprev; Uprev = U; U = tmp;
    }
    if (j->h_out) memcpy(j->h_out + bh * N * P, h, sizeof(double) * N * P);
    if (j->Bprev_out && j->xprev_out) {
        if (L > 0) {
            const int64_t last = (b * L + (L - 1)) * H + hh;
            memcpy(j->Bprev_out + bh * R * N, j->Bm + last * R * N, sizeof(double) * R * N);
            memcpy(j->xprev_out + bh * R * P, j->x + last * R * P, sizeof(double) * R * P);
        } else if (j->Bprev0 && j->xprev0) {
            memcpy(j->Bprev_out + bh * R * N, j->Bprev0 + bh * R * N, sizeof(double) * R * N);
            memcpy(j->xprev_out + bh * R * P, j->xprev0 + bh * R * P, sizeof(double) * R * P);
        } else {
            memset(j->Bprev_out + bh * R * N, 0, sizeof(double) * R * N);
            memset(j->xprev_out + bh * R * P, 0, sizeof(double) * R * P);
        }
    }
}

static void *scan_worker(void *arg)
{
    scan_job *j = (scan_job *)arg;
    const int64_t NP = j->N * j->P;
    double *buf = (double *)malloc(sizeof(double) * 3 * NP);
    if (!buf) {
        pthread_mutex_lock(&j->mu); j->status = -2; pthread_mutex_unlock(&j->mu);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&j->mu);
        const int64_t u = j->next_unit++;
        pthread_mutex_unlock(&j->mu);
        if (u >= j->Bt * j->H) break;
        scan_unit(j, u / j->H, u % j->H, buf, buf + NP, buf + 2 * NP);
    }
    free(buf);
    return NULL;
}

/*
 * Full scan over L steps for every (b, h).  Units are independent, so they are
 * spread over `nthreads` POSIX threads (<= 0 means 1).  Returns 0 on success,
 * -1 for bad sizes, -2 when memory or threads cannot be obtained.
 */
int m3o_scan(int64_t Bt, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
             const double *x, const double *Bm, const double *Cm,
             const double *dt, const double *A, const double *theta,
             const double *lam, const double *h0, const double *Bprev0,
             const double *xprev0, double *y, double *h_out,
             double *Bprev_out, double *xprev_out, int nthreads)
{
    if (Bt < 0 || L < 0 || H < 0 || P <= 0 || N <= 0 || R <= 0 || (N % 2) != 0)
        return -1;
    scan_job j = {Bt, L, H, P, N, R, x, Bm, Cm, dt, A, theta, lam,
                  h0, Bprev0, xprev0, y, h_out, Bprev_out, xprev_out, 0,
                  PTHREAD_MUTEX_INITIALIZER, 0};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, scan_worker, &j) != 0) break;
        ++started;
    }
    if (started == 0) scan_worker(&j);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    return j.status;
}

/*
 * One autoregressive step on a resident state record, for every (b, h):
 *   inputs  x_t [Bt,H,R,P], Bm_t, Cm_t [Bt,H,R,N], dt_t, lam_t [Bt,H],
 *           theta_t [Bt,H,N/2], A_t [Bt,H]
 *   in/out  h [Bt,H,N,P], Bprev [Bt,H,R,N], xprev [Bt,H,R,P]
 *   out     y_t [Bt,H,R,P]
 * This is the scan's step applied once, with the previous endpoint taken from
 * the record and the record advanced to (B_t, X_t).
 */
int m3o_decode_step(int64_t Bt, int64_t H, int64_t P, int64_t N, int64_t R,
                    const double *x, const double *Bm, const double *Cm,
                    const double *dt, const double *A, const double *theta,
                    const double *lam, double *h, double *Bprev, double *xprev,
                    double *y)
{
    if (Bt < 0 || H < 0 || P <= 0 || N <= 0 || R <= 0 || (N % 2) != 0)
        return -1;
    double *Uprev = (double *)malloc(sizeof(double) * 2 * N * P);
    if (!Uprev) return -2;
    double *U = Uprev + N * P;
    for (int64_t u = 0; u < Bt * H; ++u) {
        input_term(Bprev + u * R * N, xprev + u * R * P, N, P, R, Uprev);
        input_term(Bm + u * R * N, x + u * R * P, N, P, R, U);
        step(h + u * N * P, Uprev, U, Cm + u * R * N, dt[u], A[u],
             theta + u * (N / 2), lam[u], N, P, R, y + u * R * P);
        memcpy(Bprev + u * R * N, Bm + u * R * N, sizeof(double) * R * N);
        memcpy(xprev + u * R * P, x + u * R * P, sizeof(double) * R * P);
    }
    free(Uprev);
    return 0;
}
