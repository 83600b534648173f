/*
 * ss_oracle.c -- plain fp64 CPU reference of the selective scan and of the
 * single-token recurrent step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path links, loads or
 * calls this file; only the tests, the smoke check and the bench's CPU
 * baseline do.  It shares no code, header or table with the GPU kernels.
 *
 * What it computes (Mamba walk-through, section 3.3 "selective_scan", with
 * the shapes of its docstring; the discrete recurrence of section 2.2; the
 * D parameter and the silu(z) gate of the Mamba block, section 3.4):
 *
 *   for every lane (b, d), starting from h = h0[b, d, :] (zeros if absent):
 *     for t = 0 .. L-1:
 *       delta = Delta[b, t, d],  x = u[b, t, d]
 *       for n:  h[n] = exp(delta * A[d, n]) * h[n] + (delta * B[b, t, n]) * x
 *       y = sum_n h[n] * C[b, t, n]            (post-update state, y_t = C h_t)
 *       y += Dskip[d] * x                      (if Dskip)
 *       y *= z / (1 + exp(-z)),  z = Z[b,t,d]  (if Z: silu gate)
 *       out[b, t, d] = y
 *
 * Two options change how delta and Bbar are formed (flags):
 *  - ORACLE_SOFTPLUS, with an optional per-channel delta_bias: the step size
 *    is softplus(delta + delta_bias[d]), softplus(v) = log(1 + e^v) (LTI
 *    chapter, section 3.1.4.2: delta_t = Softplus(Parameter + projection of
 *    x_t), the Parameter being one value per channel).  A bias without the
 *    flag is added as is.
 *  - ORACLE_ZOH: Bbar = (delta*A)^-1 (exp(delta*A) - 1) * delta*B, the
 *    zero-order-hold form of the walk-through's section 2.2, elementwise for
 *    the diagonal A; at delta*A = 0 it takes its limit delta*B.
 *
 * Readings of the pages taken here (each also listed in the design notes):
 *  - Abar = exp(delta*A) (zero-order hold, section 2.2), Bbar = delta*B (the
 *    Euler form the section 3.3 code uses) unless ORACLE_ZOH, so the input
 *    term is delta*B*x.
 *  - y reads the state after the update at t.
 *  - delta arrives already positive unless ORACLE_SOFTPLUS.
 *  - A is a fixed (D, N) array; only delta, B and C vary with t.
 *  - D skip is added before the gate.
 *
 * Precision: every input is widened exactly to double (bf16 patterns are
 * shifted into the high half of a float first); all arithmetic is double,
 * libm exp, summation over n in ascending order.  Built with
 * -ffp-contract=off so no fused multiply-add changes the rounding sequence.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_MAX_N 1024
#define ORACLE_SOFTPLUS 1
#define ORACLE_ZOH 2

static double widen(const void* p, int64_t i, int dtype)
{
    if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* log(1 + e^v), written so that neither branch overflows or cancels */
static double softplus(double v) { return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v)); }

/* the step size of lane d at one timestep: raw delta, plus the channel's
 * bias, through softplus when asked */
static double step_size(double raw, const float* delta_bias, int64_t d, int flags)
{
    double v = raw + (delta_bias ? (double)delta_bias[d] : 0.0);
    return (flags & ORACLE_SOFTPLUS) ? softplus(v) : v;
}

/* Bbar[n] * x for step size delta, A[d,n] = a, B[b,t,n] = bm */
static double input_term(double delta, double a, double bm, double x, int flags)
{
    double b_bar = delta * bm; /* Euler */
    if (flags & ORACLE_ZOH) {
        const double da = delta * a;
        /* (delta*A)^-1 (exp(delta*A) - 1), continuous at delta*A = 0 */
        const double phi = da == 0.0 ? 1.0 : expm1(da) / da;
        b_bar = phi * (delta * bm);
    }
    return b_bar * x;
}

typedef struct {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* Dskip;
    const void* z;
    const double* h0;
    const float* delta_bias;
    int flags;
    int dtype;
    int64_t batch, seqlen, dim, dstate;
    const int64_t* lanes;
    int64_t n_lanes;
    double* y_out;
    double* h_last;
    const int64_t* rec_t;
    int64_t n_rec;
    double* h_rec;
} scan_job;

/* One lane (b, d) over the whole sequence. */
static void scan_lane(const scan_job* j, int64_t li)
{
    const int64_t L = j->seqlen, D = j->dim, N = j->dstate;
    const int64_t bd = j->lanes ? j->lanes[li] : li;
    const int64_t b = bd / D, d = bd % D;
    double h[ORACLE_MAX_N];
    int64_t next_rec = 0;

    for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[bd * N + n] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = (b * L + t) * D + d;  /* (B, L, D) row-major */
        const int64_t srow = (b * L + t) * N;     /* (B, L, N) row-major */
        const double delta = step_size(widen(j->delta, row, j->dtype), j->delta_bias, d, j->flags);
        const double x = widen(j->u, row, j->dtype);
        for (int64_t n = 0; n < N; ++n) {
            const double a = (double)j->A[d * N + n];
            const double a_bar = exp(delta * a);
            h[n] = a_bar * h[n] + input_term(delta, a, widen(j->B, srow + n, j->dtype), x, j->flags);
        }
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) y += h[n] * widen(j->C, srow + n, j->dtype);
        if (j->Dskip) y += (double)j->Dskip[d] * x;
        if (j->z) y *= silu(widen(j->z, row, j->dtype));
        if (j->y_out) j->y_out[li * L + t] = y;

        while (j->h_rec && next_rec < j->n_rec && j->rec_t[next_rec] == t) {
            memcpy(&j->h_rec[(li * j->n_rec + next_rec) * N], h, (size_t)N * sizeof(double));
            ++next_rec;
        }
    }
    if (j->h_last) memcpy(&j->h_last[li * N], h, (size_t)N * sizeof(double));
}

typedef struct {
    const scan_job* job;
    int64_t begin, end;
} scan_slice;

static void* scan_worker(void* arg)
{
    const scan_slice* s = (const scan_slice*)arg;
    for (int64_t li = s->begin; li < s->end; ++li) scan_lane(s->job, li);
    return NULL;
}

/*
 * oracle_scan: y_out (n_lanes, L) double, h_last (n_lanes, N) double,
 * h_rec (n_lanes, n_rec, N) double: the state right after timestep rec_t[k]
 * (rec_t ascending).  lanes: flat b*D + d indices, or NULL for all B*D lanes
 * in order.  Any output pointer may be NULL.  nthreads <= 1 runs on the
 * calling thread; otherwise lanes are split into contiguous blocks, one per
 * thread (lanes are independent, so the result does not depend on it).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_scan(const void* u, const void* delta, const float* A, const void* B, const void* C,
                const float* Dskip, const void* z, const double* h0,
                const float* delta_bias, int flags, int dtype,
                int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                const int64_t* lanes, int64_t n_lanes,
                double* y_out, double* h_last,
                const int64_t* rec_t, int64_t n_rec, double* h_rec, int nthreads)
{
    if (!u || !delta || !A || !B || !C) return -1;
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0 || dstate > ORACLE_MAX_N) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (flags & ~(ORACLE_SOFTPLUS | ORACLE_ZOH)) return -1;
    if (!lanes) n_lanes = batch * dim;
    for (int64_t i = 0; lanes && i < n_lanes; ++i)
        if (lanes[i] < 0 || lanes[i] >= batch * dim) return -1;
    for (int64_t k = 1; rec_t && k < n_rec; ++k)
        if (rec_t[k] <= rec_t[k - 1]) return -1;

    scan_job job = {u, delta, A, B, C, Dskip, z, h0, delta_bias, flags, dtype, batch, seqlen, dim, dstate,
                    lanes, n_lanes, y_out, h_last, rec_t, rec_t ? n_rec : 0, h_rec};

    if (nthreads <= 1 || n_lanes < 2) {
        for (int64_t li = 0; li < n_lanes; ++li) scan_lane(&job, li);
        return 0;
    }
    if (nthreads > n_lanes) nthreads = (int)n_lanes;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    scan_slice* sl = (scan_slice*)malloc(sizeof(scan_slice) * (size_t)nthreads);
    if (!th || !sl) {
        free(th);
        free(sl);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        sl[i].job = &job;
        sl[i].begin = n_lanes * i / nthreads;
        sl[i].end = n_lanes * (i + 1) / nthreads;
        pthread_create(&th[i], NULL, scan_worker, &sl[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(sl);
    return 0;
}

/*
 * oracle_step: one token of the recurrent mode (the walk-through's O(1)-state
 * inference, section 6; on the interactive demo page the state is all that
 * is carried from one token to the next).  h (n_lanes, N) double is read and
 * overwritten; u, delta, z are
 * (B, D), B and C are (B, N), all in `dtype`; y_out (n_lanes) double.
 * nthreads > 1 splits the lanes into contiguous blocks, one per thread; lanes
 * are independent, so the result does not depend on it.
 */
typedef struct {
    double* h;
    const void *u, *delta, *B, *C, *z;
    const float *A, *Dskip, *delta_bias;
    int flags, dtype;
    int64_t batch, dim, dstate;
    const int64_t* lanes;
    double* y_out;
} step_job;

static void step_lane(const step_job* j, int64_t li)
{
    const int64_t bd = j->lanes ? j->lanes[li] : li;
    const int64_t b = bd / j->dim, d = bd % j->dim, N = j->dstate;
    const double delta_v = step_size(widen(j->delta, bd, j->dtype), j->delta_bias, d, j->flags);
    const double x = widen(j->u, bd, j->dtype);
    double* hl = &j->h[li * N];
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double a = (double)j->A[d * N + n];
        const double a_bar = exp(delta_v * a);
        hl[n] = a_bar * hl[n] + input_term(delta_v, a, widen(j->B, b * N + n, j->dtype), x, j->flags);
    }
    for (int64_t n = 0; n < N; ++n) y += hl[n] * widen(j->C, b * N + n, j->dtype);
    if (j->Dskip) y += (double)j->Dskip[d] * x;
    if (j->z) y *= silu(widen(j->z, bd, j->dtype));
    if (j->y_out) j->y_out[li] = y;
}

typedef struct {
    const step_job* job;
    int64_t begin, end;
} step_slice;

static void* step_worker(void* arg)
{
    const step_slice* s = (const step_slice*)arg;
    for (int64_t li = s->begin; li < s->end; ++li) step_lane(s->job, li);
    return NULL;
}

int oracle_step(double* h, const void* u, const void* delta, const float* A, const void* B,
                const void* C, const float* Dskip, const void* z,
                const float* delta_bias, int flags, int dtype,
                int64_t batch, int64_t dim, int64_t dstate,
                const int64_t* lanes, int64_t n_lanes, double* y_out, int nthreads)
{
    if (!h || !u || !delta || !A || !B || !C) return -1;
    if (batch <= 0 || dim <= 0 || dstate <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (flags & ~(ORACLE_SOFTPLUS | ORACLE_ZOH)) return -1;
    if (!lanes) n_lanes = batch * dim;
    for (int64_t li = 0; lanes && li < n_lanes; ++li)
        if (lanes[li] < 0 || lanes[li] >= batch * dim) return -1;
    step_job job = {h, u, delta, B, C, z, A, Dskip, delta_bias, flags, dtype, batch, dim, dstate, lanes, y_out};
    if (nthreads <= 1 || n_lanes < 2) {
        for (int64_t li = 0; li < n_lanes; ++li) step_lane(&job, li);
        return 0;
    }
    if (nthreads > n_lanes) nthreads = (int)n_lanes;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    step_slice* sl = (step_slice*)malloc(sizeof(step_slice) * (size_t)nthreads);
    if (!th || !sl) {
        free(th);
        free(sl);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        sl[i].job = &job;
        sl[i].begin = n_lanes * i / nthreads;
        sl[i].end = n_lanes * (i + 1) / nthreads;
        pthread_create(&th[i], NULL, step_worker, &sl[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(sl);
    return 0;
}

/*
 * Backward of the scan: the gradients of
 *   Loss = sum_{b,t,d} dy[b,t,d] * out[b,t,d] + sum_{b,d,n} dh_last[b,d,n] * h_last[b,d,n]
 * with respect to every input of oracle_scan, by the chain rule taken backward
 * through the forward recurrence (the backward that the walk-through's
 * section 3.3 and the LTI chapter's section 3.1.5.3 say recomputes the states
 * from the inputs instead of storing them):
 *
 *   per lane (b, d): run the forward once, keeping every state h_t, the step
 *   sizes and the pre-gate outputs; then with g = dh_last (0 if absent), for
 *   t = L-1 down to 0:
 *     gate:   dz_t = dy_t * ypre_t * silu'(z_t);  dy_t <- dy_t * silu(z_t)
 *     skip:   du_t += dy_t * D[d];  dD[d] += dy_t * u_t
 *     output: dC[b,t,n] += dy_t * h_t[n];  g[n] += dy_t * C[b,t,n]
 *     update h_t[n] = e[n] h_{t-1}[n] + beta[n] B[b,t,n] u_t,  e[n] = exp(delta_t A[d,n]),
 *             beta[n] the input coefficient (see input_coef):
 *             ddelta_t += g[n] (A[d,n] e[n] h_{t-1}[n] + dbeta/ddelta B[b,t,n] u_t)
 *             dA[d,n]  += g[n] (delta_t e[n] h_{t-1}[n] + dbeta/dA B[b,t,n] u_t)
 *             dB[b,t,n] += g[n] beta[n] u_t;  du_t += g[n] beta[n] B[b,t,n]
 *             g[n] <- g[n] e[n]
 *     step size: with softplus, d(raw)_t = ddelta_t * sigmoid(raw_t + bias[d]);
 *             dbias[d] += d(raw)_t (a bias enters with derivative 1)
 *   dh0 = g.
 * silu'(z) = s (1 + z (1 - s)), s = sigmoid(z).
 *
 * dA, dD, dbias sum over batch rows and dB, dC over channels.  The lanes are
 * cut into at most 64 fixed blocks, each block adds its lanes' terms in lane
 * order into its own accumulators, and the blocks are added in block order:
 * the result does not depend on the thread count.
 */
#define BWD_MAX_BLOCKS 64

typedef struct {
    const scan_job* f;
    const double* dy;
    const double* dh_last;
    double *du, *ddelta, *dz, *dh0; /* per lane, written directly */
    int64_t nblk;
    double* acc; /* nblk blocks of [dA (D*N) | dD (D) | dbias (D) | dB (B*L*N) | dC (B*L*N)] */
    int64_t acc_stride;
} bwd_job;

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/*
 * The input coefficient beta, Bbar = beta * B, and its partial derivatives,
 * for step size delta and A[d,n] = a (the discretisations of the
 * walk-through's section 2.2):
 *  - Euler: beta = delta; dbeta/ddelta = 1, dbeta/da = 0.
 *  - zero-order hold: beta = (e^x - 1) / a = delta phi(x), x = delta a,
 *    phi(x) = (e^x - 1) / x (1 at x = 0).  Then dbeta/ddelta = e^x (also at
 *    a = 0, where beta = delta), and dbeta/da = delta^2 psi(x) with
 *    psi(x) = phi'(x) = (x e^x - e^x + 1) / x^2, psi(0) = 1/2.  Near 0 the
 *    closed form cancels, so psi comes from its Taylor series
 *    sum_k (k + 1) x^k / (k + 2)! (the series of e^x, shifted twice).
 */
static void input_coef(double delta, double a, int flags, double* beta, double* dbeta_ddelta, double* dbeta_da)
{
    if (!(flags & ORACLE_ZOH)) {
        *beta = delta;
        *dbeta_ddelta = 1.0;
        *dbeta_da = 0.0;
        return;
    }
    const double x = delta * a;
    const double phi = x == 0.0 ? 1.0 : expm1(x) / x;
    double psi;
    if (fabs(x) < 0.01) {
        double xk = 1.0, fact = 2.0; /* x^k and (k + 2)! */
        psi = 0.0;
        for (int k = 0; k < 10; ++k) {
            psi += (double)(k + 1) * xk / fact;
            xk *= x;
            fact *= (double)(k + 3);
        }
    } else {
        psi = (x * exp(x) - expm1(x)) / (x * x);
    }
    *beta = phi * delta;
    *dbeta_ddelta = exp(x);
    *dbeta_da = delta * delta * psi;
}

static void bwd_lane(const bwd_job* j, int64_t bd, double* hs, double* acc)
{
    const scan_job* f = j->f;
    const int64_t L = f->seqlen, D = f->dim, N = f->dstate;
    const int64_t b = bd / D, d = bd % D;
    double* dA = acc;
    double* dD = dA + D * N;
    double* dbias = dD + D;
    double* dB = dbias + D;
    double* dC = dB + f->batch * L * N;
    double* dl = hs + (L + 1) * N; /* step sizes */
    double* yp = dl + L;           /* pre-gate outputs */

    for (int64_t n = 0; n < N; ++n) hs[n] = f->h0 ? f->h0[bd * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = (b * L + t) * D + d, srow = (b * L + t) * N;
        const double delta = step_size(widen(f->delta, row, f->dtype), f->delta_bias, d, f->flags);
        const double x = widen(f->u, row, f->dtype);
        const double* hp = hs + t * N;
        double* hn = hs + (t + 1) * N;
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double a = (double)f->A[d * N + n];
            hn[n] = exp(delta * a) * hp[n] + input_term(delta, a, widen(f->B, srow + n, f->dtype), x, f->flags);
        }
        for (int64_t n = 0; n < N; ++n) y += hn[n] * widen(f->C, srow + n, f->dtype);
        if (f->Dskip) y += (double)f->Dskip[d] * x;
        dl[t] = delta;
        yp[t] = y;
    }

    double g[ORACLE_MAX_N];
    for (int64_t n = 0; n < N; ++n) g[n] = j->dh_last ? j->dh_last[bd * N + n] : 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t row = (b * L + t) * D + d, srow = (b * L + t) * N;
        const double x = widen(f->u, row, f->dtype);
        const double delta = dl[t];
        double dyt = j->dy[row];
        double du = 0.0, dd = 0.0;
        if (f->z) {
            const double zz = widen(f->z, row, f->dtype), s = sigmoid(zz);
            j->dz[row] = dyt * yp[t] * s * (1.0 + zz * (1.0 - s));
            dyt *= zz * s;
        }
        if (f->Dskip) {
            du += dyt * (double)f->Dskip[d];
            dD[d] += dyt * x;
        }
        const double* hcur = hs + (t + 1) * N;
        const double* hprev = hs + t * N;
        for (int64_t n = 0; n < N; ++n) {
            dC[srow + n] += dyt * hcur[n];
            g[n] += dyt * widen(f->C, srow + n, f->dtype);
        }
        for (int64_t n = 0; n < N; ++n) {
            const double a = (double)f->A[d * N + n];
            const double bm = widen(f->B, srow + n, f->dtype);
            const double e = exp(delta * a);
            double beta, dbeta_dd, dbeta_da;
            input_coef(delta, a, f->flags, &beta, &dbeta_dd, &dbeta_da);
            dd += g[n] * (a * e * hprev[n] + dbeta_dd * bm * x);
            dA[d * N + n] += g[n] * (delta * e * hprev[n] + dbeta_da * bm * x);
            dB[srow + n] += g[n] * beta * x;
            du += g[n] * beta * bm;
            g[n] *= e;
        }
        if (f->flags & ORACLE_SOFTPLUS) {
            const double v = widen(f->delta, row, f->dtype) + (f->delta_bias ? (double)f->delta_bias[d] : 0.0);
            dd *= sigmoid(v);
        }
        if (f->delta_bias) dbias[d] += dd;
        j->du[row] = du;
        j->ddelta[row] = dd;
    }
    for (int64_t n = 0; n < N; ++n) j->dh0[bd * N + n] = g[n];
}

typedef struct {
    const bwd_job* job;
    int first, step; /* blocks first, first + step, ... */
    int failed;
} bwd_worker_arg;

static void* bwd_worker(void* arg)
{
    bwd_worker_arg* w = (bwd_worker_arg*)arg;
    const bwd_job* j = w->job;
    const scan_job* f = j->f;
    const int64_t BD = f->batch * f->dim;
    double* hs = (double*)malloc(sizeof(double) * (size_t)((f->seqlen + 1) * f->dstate + 2 * f->seqlen));
    if (!hs) {
        w->failed = 1;
        return NULL;
    }
    for (int64_t k = w->first; k < j->nblk; k += w->step) {
        double* acc = j->acc + k * j->acc_stride;
        for (int64_t bd = BD * k / j->nblk; bd < BD * (k + 1) / j->nblk; ++bd) bwd_lane(j, bd, hs, acc);
    }
    free(hs);
    return NULL;
}

/*
 * oracle_scan_bwd: inputs as oracle_scan (all lanes), dy (B,L,D) and dh_last
 * (B,D,N, or NULL) as double.  Outputs (double, none may be NULL):
 * du, ddelta, dz (B,L,D) -- dz untouched without z; dA (D,N); dB, dC (B,L,N);
 * dD (D) -- zeros without D; dbias (D) -- zeros without a bias; dh0 (B,D,N).
 * ddelta is the gradient with respect to the delta argument as passed (the
 * raw value when ORACLE_SOFTPLUS is set).  Returns 0, or -1 on a bad argument,
 * an unknown option or a failed allocation.
 */
int oracle_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                    const float* Dskip, const void* z, const double* h0,
                    const float* delta_bias, int flags, int dtype,
                    int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    const double* dy, const double* dh_last,
                    double* du, double* ddelta, double* dz, double* dA, double* dB, double* dC,
                    double* dD, double* dbias, double* dh0, int nthreads)
{
    if (!u || !delta || !A || !B || !C || !dy) return -1;
    if (!du || !ddelta || !dz || !dA || !dB || !dC || !dD || !dbias || !dh0) return -1;
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0 || dstate > ORACLE_MAX_N) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (flags & ~(ORACLE_SOFTPLUS | ORACLE_ZOH)) return -1;
    const int64_t BD = batch * dim, L = seqlen, N = dstate, D = dim;

    scan_job f = {u, delta, A, B, C, Dskip, z, h0, delta_bias, flags, dtype, batch, seqlen, dim, dstate,
                  NULL, BD, NULL, NULL, NULL, 0, NULL};
    bwd_job job = {&f, dy, dh_last, du, ddelta, dz, dh0, BD < BWD_MAX_BLOCKS ? BD : BWD_MAX_BLOCKS, NULL, 0};
    job.acc_stride = D * N + 2 * D + 2 * batch * L * N;
    job.acc = (double*)calloc((size_t)(job.nblk * job.acc_stride), sizeof(double));
    if (!job.acc) return -1;

    if (nthreads < 1) nthreads = 1;
    if (nthreads > job.nblk) nthreads = (int)job.nblk;
    pthread_t th[BWD_MAX_BLOCKS];
    bwd_worker_arg wa[BWD_MAX_BLOCKS];
    for (int i = 0; i < nthreads; ++i) {
        wa[i].job = &job;
        wa[i].first = i;
        wa[i].step = nthreads;
        wa[i].failed = 0;
    }
    if (nthreads == 1) {
        bwd_worker(&wa[0]);
    } else {
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bwd_worker, &wa[i]);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i)
        if (wa[i].failed) rc = -1;

    /* blocks added in block order */
    memset(dA, 0, sizeof(double) * (size_t)(D * N));
    memset(dD, 0, sizeof(double) * (size_t)D);
    memset(dbias, 0, sizeof(double) * (size_t)D);
    memset(dB, 0, sizeof(double) * (size_t)(batch * L * N));
    memset(dC, 0, sizeof(double) * (size_t)(batch * L * N));
    for (int64_t k = 0; k < job.nblk; ++k) {
        const double* acc = job.acc + k * job.acc_stride;
        for (int64_t i = 0; i < D * N; ++i) dA[i] += acc[i];
        for (int64_t i = 0; i < D; ++i) dD[i] += acc[D * N + i];
        for (int64_t i = 0; i < D; ++i) dbias[i] += acc[D * N + D + i];
        for (int64_t i = 0; i < batch * L * N; ++i) dB[i] += acc[D * N + 2 * D + i];
        for (int64_t i = 0; i < batch * L * N; ++i) dC[i] += acc[D * N + 2 * D + batch * L * N + i];
    }
    free(job.acc);
    return rc;
}

/*
 * oracle_conv1d_silu: the Mamba block's causal depthwise convolution and
 * SiLU that produce the scan's input u (walk-through, section 3.4: a Conv1d
 * with one filter per channel, padding width-1 and only the first L outputs
 * kept, then silu):
 *   u[b,t,d] = silu(bias[d] + sum_{k=0}^{width-1} w[d,k] * x[b, t-width+1+k, d]),
 * with x = 0 before t = 0.  x rows are x_row_stride elements apart (x may be
 * the first half of a (B, L, 2D) projection read in place); w is (D, width)
 * fp32, bias (D) fp32 or NULL.  u_out (B, L, D) double.  Returns 0 or -1.
 */
int oracle_conv1d_silu(const void* x, int64_t x_row_stride, const float* w, const float* bias, int dtype,
                       int64_t batch, int64_t seqlen, int64_t dim, int64_t width, double* u_out)
{
    if (!x || !w || !u_out) return -1;
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || width <= 0 || x_row_stride < dim) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t t = 0; t < seqlen; ++t)
            for (int64_t d = 0; d < dim; ++d) {
                double acc = bias ? (double)bias[d] : 0.0;
                for (int64_t k = 0; k < width; ++k) {
                    const int64_t s = t - width + 1 + k;
                    if (s < 0) continue;
                    acc += (double)w[d * width + k] * widen(x, (b * seqlen + s) * x_row_stride + d, dtype);
                }
                u_out[(b * seqlen + t) * dim + d] = silu(acc);
            }
    return 0;
}

/*
 * oracle_ssd: the multi-head state-space recurrence of Mamba-2 (walk-through,
 * section 4.1: h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t, with a state per
 * head; section 5.2: heads of headdim channels and d_state up to 128-256).
 * Per batch row b and head h the state S is (N, P):
 *   S_t = exp(dt[b,t,h] * A[h]) S_{t-1} + dt[b,t,h] * B[b,t,:] (outer) x[b,t,h,:]
 *   y[b,t,h,:] = S_t^T C[b,t,:] + D[h] x[b,t,h,:]
 * A_t = exp(dt A) with a scalar A per head and the input term dt*B*x are
 * the discretisation of section 2.2 (the same as oracle_scan's) applied per
 * head; B and C are shared by all heads.  x, y (B, L, H, P); dt (B, L, H);
 * B, C (B, L, N), all in `dtype`; A, D (H) fp32 (D may be NULL); h0 (B, H, N,
 * P) double or NULL.  Outputs (double): y_out (B, L, H, P), h_last (B, H, N,
 * P), either may be NULL.  heads: NULL for all (b, h) pairs in order, or a
 * list of flat b*H + h (then y_out is (n, L, P) and h_last (n, N, P)).
 * nthreads > 1 splits the (b, h) pairs into contiguous blocks, one per
 * thread; pairs are independent, so the result does not depend on it.
 * Returns 0 or -1.
 */
typedef struct {
    const void *x, *dt, *B, *C;
    const float *A, *D;
    const double* h0;
    int dtype;
    int64_t batch, seqlen, heads, hdim, dstate;
    const int64_t* sel;
    double *y_out, *h_last;
} ssd_job;

/* one (b, h) pair, k-th of the selection; S is an (N, P) scratch state */
static void ssd_pair(const ssd_job* j, int64_t k, double* S)
{
    const int64_t L = j->seqlen, H = j->heads, P = j->hdim, N = j->dstate;
    const int64_t bh = j->sel ? j->sel[k] : k;
    const int64_t b = bh / H, h = bh % H;
    for (int64_t i = 0; i < N * P; ++i) S[i] = j->h0 ? j->h0[bh * N * P + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const double d = widen(j->dt, (b * L + t) * H + h, j->dtype);
        const double a = exp(d * (double)j->A[h]);
        const int64_t xrow = ((b * L + t) * H + h) * P, srow = (b * L + t) * N;
        for (int64_t n = 0; n < N; ++n) {
            const double bn = widen(j->B, srow + n, j->dtype);
            for (int64_t p = 0; p < P; ++p) S[n * P + p] = a * S[n * P + p] + d * bn * widen(j->x, xrow + p, j->dtype);
        }
        for (int64_t p = 0; p < P; ++p) {
            double y = 0.0;
            for (int64_t n = 0; n < N; ++n) y += S[n * P + p] * widen(j->C, srow + n, j->dtype);
            if (j->D) y += (double)j->D[h] * widen(j->x, xrow + p, j->dtype);
            if (j->y_out) j->y_out[(k * L + t) * P + p] = y;
        }
    }
    if (j->h_last) memcpy(&j->h_last[k * N * P], S, sizeof(double) * (size_t)(N * P));
}

typedef struct {
    const ssd_job* job;
    int64_t begin, end;
    int rc;
} ssd_slice;

static void* ssd_worker(void* arg)
{
    ssd_slice* s = (ssd_slice*)arg;
    double* S = (double*)malloc(sizeof(double) * (size_t)(s->job->dstate * s->job->hdim));
    if (!S) {
        s->rc = -1;
        return NULL;
    }
    for (int64_t k = s->begin; k < s->end; ++k) ssd_pair(s->job, k, S);
    free(S);
    s->rc = 0;
    return NULL;
}

int oracle_ssd(const void* x, const void* dt, const float* A, const void* B, const void* C, const float* D,
               const double* h0, int dtype, int64_t batch, int64_t seqlen, int64_t heads, int64_t hdim,
               int64_t dstate, const int64_t* sel, int64_t n_sel, double* y_out, double* h_last, int nthreads)
{
    if (!x || !dt || !A || !B || !C) return -1;
    if (batch <= 0 || seqlen <= 0 || heads <= 0 || hdim <= 0 || dstate <= 0) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (!sel) n_sel = batch * heads;
    for (int64_t k = 0; sel && k < n_sel; ++k)
        if (sel[k] < 0 || sel[k] >= batch * heads) return -1;
    ssd_job job = {x, dt, B, C, A, D, h0, dtype, batch, seqlen, heads, hdim, dstate, sel, y_out, h_last};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_sel) nthreads = (int)(n_sel > 0 ? n_sel : 1);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    ssd_slice* sl = (ssd_slice*)malloc(sizeof(ssd_slice) * (size_t)nthreads);
    if (!th || !sl) {
        free(th);
        free(sl);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        sl[i].job = &job;
        sl[i].begin = n_sel * i / nthreads;
        sl[i].end = n_sel * (i + 1) / nthreads;
        sl[i].rc = 0;
    }
    if (nthreads == 1) {
        ssd_worker(&sl[0]);
    } else {
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, ssd_worker, &sl[i]);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    }
    int rc = 0;
    for (int i = 0; i < nthreads; ++i)
        if (sl[i].rc != 0) rc = -1;
    free(th);
    free(sl);
    return rc;
}
