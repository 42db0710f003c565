/*
 * ssm_oracle.c -- plain f64 CPU oracle of the Mamba S6 selective scan.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library; nothing in the product path calls it.
 *
 * What it computes (rustytorch commit log, page "crates/training/rtx-transformers/
 * tests", commit that replaces the MambaBlock stub with a real S6 forward):
 *   A      = -exp(A_log)                              per (channel d, state n)
 *   delta  = softplus(dt + dt_bias)                   per (b, t, d), stable form
 *   h_t    = exp(delta*A) * h_{t-1} + delta*B_t*x_t   per (b, d, n), sequential in t
 *   ypre_t = sum_n C_t[n]*h_t[n] + D*x_t
 *   y_t    = ypre_t * silu(z_t)                       (no gate when z is NULL)
 * B_t and C_t are per token and shared by every channel (the x_proj of that
 * commit emits 2*d_state values per token).  The discretised input term is read
 * as delta*B_t*x_t (Euler form); the zero-order-hold form is not used.
 *
 * The backward (same log, commit adding the hand-written VJP) is the
 * reverse-time adjoint recurrence over the recomputed state trajectory; the
 * gradient for A_log goes through dA_log = dA * A; parameter gradients
 * (A_log, D, dt_bias) are summed over batch and time, dB/dC over channels.
 *
 * The single-token step (commit introducing MambaRecurrence::step) applies the
 * forward's per-token body to a caller-held state; stepping from a zero state
 * reproduces the forward exactly because both call token_update() below.
 *
 * Layouts (dense, row-major, last index fastest):
 *   x, dt, z, y, dy, dx, ddt, dz, ddelta : [Bt, L, D]
 *   B, C, dB, dC                         : [Bt, L, N]
 *   A_log, dA_log                        : [D, N]
 *   Dp, dt_bias, dD, ddt_bias            : [D]
 *   h0, h_last, dh0, step state h        : [Bt, D, N]
 * Nullable inputs: z (no gate), Dp (D = 0), dt_bias (0), h0 (zero state).
 * Nullable outputs: h_last, delta_out, dz (required when z != NULL), dh0, ddelta.
 *
 * Parallelism: OpenMP over fixed blocks of channels.  Per-(b,t,n) sums over
 * channels (dB, dC) go to per-block buffers summed in block order, so results
 * do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DBLOCK 16 /* channels per work block */

static double softplus_d(double u) {
    /* stable softplus: log(1 + e^u) without overflow */
    return u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u));
}

static double sigmoid_d(double z) {
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

/* One token of one channel.  h[N] is updated in place; returns ypre (before
 * the gate) and writes delta to *delta_out.  Used by the full forward, the
 * backward's recompute and the single-token step. */
static double token_update(int64_t N, const double *A, double *h, double xv, double dtv,
                           double bias, double Dd, const double *Bt, const double *Ct,
                           double *delta_out) {
    double delta = softplus_d(dtv + bias);
    double dx = delta * xv;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double a = exp(delta * A[n]);
        h[n] = a * h[n] + dx * Bt[n];
        acc += Ct[n] * h[n];
    }
    *delta_out = delta;
    return acc + Dd * xv;
}

static double gate(double ypre, const double *z, int64_t i) {
    if (!z) return ypre;
    double zv = z[i];
    return ypre * (zv * sigmoid_d(zv));
}

static void load_A(int64_t N, const double *A_log, int64_t d, double *A) {
    for (int64_t n = 0; n < N; ++n) A[n] = -exp(A_log[d * N + n]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_fwd(int64_t Bt, int64_t L, int64_t D, int64_t N, const double *x, const double *dt,
               const double *B, const double *C, const double *z, const double *A_log,
               const double *Dp, const double *dt_bias, const double *h0, double *y,
               double *h_last, double *delta_out) {
    if (Bt <= 0 || L < 0 || D <= 0 || N <= 0) return 2;
    int64_t nch = Bt * D;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nch; ++c) {
        int64_t b = c / D, d = c % D;
        double *A = (double *)malloc(sizeof(double) * (size_t)N);
        double *h = (double *)malloc(sizeof(double) * (size_t)N);
        load_A(N, A_log, d, A);
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
        double bias = dt_bias ? dt_bias[d] : 0.0;
        double Dd = Dp ? Dp[d] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            int64_t i = (b * L + t) * D + d;
            const double *Bt_ = B + (b * L + t) * N;
            const double *Ct_ = C + (b * L + t) * N;
            double delta;
            double ypre = token_update(N, A, h, x[i], dt[i], bias, Dd, Bt_, Ct_, &delta);
            y[i] = gate(ypre, z, i);
            if (delta_out) delta_out[i] = delta;
        }
        if (h_last)
            for (int64_t n = 0; n < N; ++n) h_last[(b * D + d) * N + n] = h[n];
        free(A);
        free(h);
    }
    return 0;
}

int oracle_step(int64_t Bt, int64_t D, int64_t N, double *h, const double *x, const double *dt,
                const double *B, const double *C, const double *z, const double *A_log,
                const double *Dp, const double *dt_bias, double *y) {
    if (Bt <= 0 || D <= 0 || N <= 0) return 2;
    int64_t nch = Bt * D;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nch; ++c) {
        int64_t b = c / D, d = c % D;
        double *A = (double *)malloc(sizeof(double) * (size_t)N);
        load_A(N, A_log, d, A);
        double bias = dt_bias ? dt_bias[d] : 0.0;
        double Dd = Dp ? Dp[d] : 0.0;
        int64_t i = b * D + d;
        double delta;
        double ypre = token_update(N, A, h + i * N, x[i], dt[i], bias, Dd, B + b * N, C + b * N,
                                   &delta);
        y[i] = gate(ypre, z, i);
        free(A);
    }
    return 0;
}

/* Reverse-time adjoint of one channel (b, d).  lam[n] carries dL/dh_t[n]. */
static void bwd_channel(int64_t Bt, int64_t L, int64_t D, int64_t N, int64_t b, int64_t d,
                        const double *x, const double *dt, const double *B, const double *C,
                        const double *z, const double *A, double bias, double Dd,
                        const double *h0, const double *dy, double *dx, double *ddt,
                        double *dz, double *ddelta, double *dBblk, double *dCblk,
                        double *dA_acc, double *dD_acc, double *ddtb_acc, double *dh0,
                        double *H /* (L+1)*N scratch */, double *lam) {
    (void)Bt;
    /* recompute the state trajectory: H[t+1] = h_t, H[0] = h_{-1} */
    for (int64_t n = 0; n < N; ++n) H[n] = h0 ? h0[(b * D + d) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        int64_t i = (b * L + t) * D + d;
        memcpy(H + (t + 1) * N, H + t * N, sizeof(double) * (size_t)N);
        double delta;
        token_update(N, A, H + (t + 1) * N, x[i], dt[i], bias, Dd, B + (b * L + t) * N,
                     C + (b * L + t) * N, &delta);
    }
    for (int64_t n = 0; n < N; ++n) lam[n] = 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
        int64_t i = (b * L + t) * D + d;
        const double *Bt_ = B + (b * L + t) * N;
        const double *Ct_ = C + (b * L + t) * N;
        const double *hprev = H + t * N;     /* h_{t-1} */
        const double *hcur = H + (t + 1) * N; /* h_t */
        double u = dt[i] + bias;
        double delta = softplus_d(u);
        double xv = x[i];
        double ypre = Dd * xv;
        for (int64_t n = 0; n < N; ++n) ypre += Ct_[n] * hcur[n];
        double g; /* dL/dypre */
        if (z) {
            double zv = z[i], s = sigmoid_d(zv);
            g = dy[i] * zv * s;
            dz[i] = dy[i] * ypre * s * (1.0 + zv * (1.0 - s));
        } else {
            g = dy[i];
        }
        *dD_acc += g * xv;
        double dxv = g * Dd;
        double dd = 0.0;
        double *dBrow = dBblk + (b * L + t) * N;
        double *dCrow = dCblk + (b * L + t) * N;
        for (int64_t n = 0; n < N; ++n) {
            double a = exp(delta * A[n]);
            lam[n] += Ct_[n] * g;            /* lam = dL/dh_t */
            dCrow[n] += g * hcur[n];
            dBrow[n] += lam[n] * delta * xv;
            dxv += lam[n] * delta * Bt_[n];
            dd += lam[n] * (A[n] * a * hprev[n] + Bt_[n] * xv);
            dA_acc[n] += lam[n] * delta * a * hprev[n];
            lam[n] *= a;                      /* -> contribution to dL/dh_{t-1} */
        }
        dx[i] = dxv;
        if (ddelta) ddelta[i] = dd;
        double gdt = dd * sigmoid_d(u); /* softplus'(u) = sigmoid(u) */
        ddt[i] = gdt;
        *ddtb_acc += gdt;
    }
    if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * D + d) * N + n] = lam[n];
}

int oracle_bwd(int64_t Bt, int64_t L, int64_t D, int64_t N, const double *x, const double *dt,
               const double *B, const double *C, const double *z, const double *A_log,
               const double *Dp, const double *dt_bias, const double *h0, const double *dy,
               double *dx, double *ddt, double *dB, double *dC, double *dz, double *dA_log,
               double *dD, double *ddt_bias, double *dh0, double *ddelta) {
    if (Bt <= 0 || L < 0 || D <= 0 || N <= 0) return 2;
    if (z && !dz) return 1;
    int64_t nblk = (D + ORACLE_DBLOCK - 1) / ORACLE_DBLOCK;
    size_t rowsz = (size_t)(Bt * L * N);
    double *dBblk = (double *)calloc((size_t)nblk * rowsz, sizeof(double));
    double *dCblk = (double *)calloc((size_t)nblk * rowsz, sizeof(double));
    if (!dBblk || !dCblk) {
        free(dBblk);
        free(dCblk);
        return 5;
    }
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < nblk; ++blk) {
        double *A = (double *)malloc(sizeof(double) * (size_t)N);
        double *lam = (double *)malloc(sizeof(double) * (size_t)N);
        double *dA = (double *)malloc(sizeof(double) * (size_t)N);
        double *H = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
        int64_t d1 = (blk + 1) * ORACLE_DBLOCK < D ? (blk + 1) * ORACLE_DBLOCK : D;
        for (int64_t d = blk * ORACLE_DBLOCK; d < d1; ++d) {
            load_A(N, A_log, d, A);
            double bias = dt_bias ? dt_bias[d] : 0.0;
            double Dd = Dp ? Dp[d] : 0.0;
            double dD_acc = 0.0, ddtb_acc = 0.0;
            for (int64_t n = 0; n < N; ++n) dA[n] = 0.0;
            for (int64_t b = 0; b < Bt; ++b)
                bwd_channel(Bt, L, D, N, b, d, x, dt, B, C, z, A, bias, Dd, h0, dy, dx, ddt, dz,
                            ddelta, dBblk + blk * rowsz, dCblk + blk * rowsz, dA, &dD_acc,
                            &ddtb_acc, dh0, H, lam);
            for (int64_t n = 0; n < N; ++n) dA_log[d * N + n] = dA[n] * A[n]; /* dA_log = dA*A */
            dD[d] = dD_acc;
            ddt_bias[d] = ddtb_acc;
        }
        free(A);
        free(lam);
        free(dA);
        free(H);
    }
    /* fixed-order sum over channel blocks */
    for (size_t r = 0; r < rowsz; ++r) {
        double sb = 0.0, sc = 0.0;
        for (int64_t blk = 0; blk < nblk; ++blk) {
            sb += dBblk[blk * rowsz + r];
            sc += dCblk[blk * rowsz + r];
        }
        dB[r] = sb;
        dC[r] = sc;
    }
    free(dBblk);
    free(dCblk);
    return 0;
}
