/*
 * f64 CPU oracle of the causal depthwise conv1d + SiLU that feeds the Mamba S6
 * scan (forward, its exact adjoint, and the one-token step over a ring of the
 * last K-1 inputs).
 *
 * TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg use this file.  It shares no code with the HIP library.
 *
 * Definition followed (rustytorch commit log, page "crates/training/
 * rtx-transformers/tests"): the commit that replaces the MambaBlock stub runs
 * in_proj, then a causal depthwise conv1d, then SiLU, before x_proj and the scan;
 * the hand-written VJP commit returns gradients for conv1d_weight and
 * conv1d_bias; MambaRecurrence::step carries the recurrent state (h, conv-ring)
 * from token to token.  The pages give neither the kernel width nor the tap
 * order; read here as PyTorch's Conv1d(groups=d_inner, padding=K-1) truncated to
 * the first L outputs, i.e.
 *
 *     pre[b,t,d] = bias[d] + sum_{k=0}^{K-1} w[d,k] * v[b, t-(K-1)+k, d]
 *     y[b,t,d]   = silu(pre) = pre * sigmoid(pre)
 *
 * where v[b,tau,d] = x[b,tau,d] for tau >= 0 and, for -(K-1) <= tau < 0, the
 * caller's initial ring s0[b,d,tau+K-1] (zero when no ring is given).  The ring
 * after the sequence holds the last K-1 inputs, oldest first.  The sum starts at
 * the bias and adds the taps in increasing k, in the forward and in the step, so
 * that stepping reproduces the forward bit for bit.
 *
 * Layouts: x, y, dx, dy [Bt, L, D]; w, dw [D, K]; bias, dbias [D];
 * rings [Bt, D, K-1].  Reductions over (b, t) for dw and dbias run per channel in
 * increasing (b, t) order, so results do not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static double sigmoid(double p) {
    if (p >= 0.0) return 1.0 / (1.0 + exp(-p));
    const double e = exp(p);
    return e / (1.0 + e);
}

/* input value at time tau (may be negative: then it comes from the initial ring) */
static double tap_value(const double* x, const double* s0, int64_t b, int64_t tau, int64_t d,
                        int64_t L, int64_t D, int64_t K) {
    if (tau >= 0) return x[(b * L + tau) * D + d];
    if (!s0) return 0.0;
    return s0[(b * D + d) * (K - 1) + (tau + K - 1)];
}

static double pre_activation(const double* x, const double* w, const double* bias, const double* s0,
                             int64_t b, int64_t t, int64_t d, int64_t L, int64_t D, int64_t K) {
    double acc = bias ? bias[d] : 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += w[d * K + k] * tap_value(x, s0, b, t - (K - 1) + k, d, L, D, K);
    return acc;
}

int oracle_conv_fwd(int64_t Bt, int64_t L, int64_t D, int64_t K, const double* x, const double* w,
                    const double* bias, const double* s0, double* y, double* s_last, double* pre_out) {
    if (Bt <= 0 || L < 0 || D <= 0 || K <= 0 || !x || !w || !y) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t b = 0; b < Bt; ++b) {
            for (int64_t t = 0; t < L; ++t) {
                const double p = pre_activation(x, w, bias, s0, b, t, d, L, D, K);
                const int64_t o = (b * L + t) * D + d;
                y[o] = p * sigmoid(p);
                if (pre_out) pre_out[o] = p;
            }
            if (s_last)
                for (int64_t j = 0; j < K - 1; ++j)
                    s_last[(b * D + d) * (K - 1) + j] = tap_value(x, s0, b, L - (K - 1) + j, d, L, D, K);
        }
    }
    return 0;
}

/* Exact adjoint of oracle_conv_fwd.  dw and dbias are overwritten (summed over
 * batch and time); ds0 (may be NULL) receives the gradient of the initial ring. */
int oracle_conv_bwd(int64_t Bt, int64_t L, int64_t D, int64_t K, const double* x, const double* w,
                    const double* bias, const double* s0, const double* dy, double* dx, double* dw,
                    double* dbias, double* ds0) {
    if (Bt <= 0 || L < 0 || D <= 0 || K <= 0 || !x || !w || !dy || !dx || !dw || !dbias) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t k = 0; k < K; ++k) dw[d * K + k] = 0.0;
        dbias[d] = 0.0;
        for (int64_t b = 0; b < Bt; ++b) {
            for (int64_t t = 0; t < L; ++t) dx[(b * L + t) * D + d] = 0.0;
            if (ds0)
                for (int64_t j = 0; j < K - 1; ++j) ds0[(b * D + d) * (K - 1) + j] = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const double p = pre_activation(x, w, bias, s0, b, t, d, L, D, K);
                const double s = sigmoid(p);
                const double g = dy[(b * L + t) * D + d] * s * (1.0 + p * (1.0 - s));  /* d silu / d pre */
                dbias[d] += g;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t tau = t - (K - 1) + k;
                    dw[d * K + k] += g * tap_value(x, s0, b, tau, d, L, D, K);
                    if (tau >= 0) dx[(b * L + tau) * D + d] += w[d * K + k] * g;
                    else if (ds0) ds0[(b * D + d) * (K - 1) + (tau + K - 1)] += w[d * K + k] * g;
                }
            }
        }
    }
    return 0;
}

/* One token: y = silu(bias + sum_k w[k] * v_k) with v_0..v_{K-2} the ring (oldest
 * first) and v_{K-1} = x; then the ring drops its oldest entry and appends x. */
int oracle_conv_step(int64_t Bt, int64_t D, int64_t K, double* ring, const double* x, const double* w,
                     const double* bias, double* y) {
    if (Bt <= 0 || D <= 0 || K <= 0 || !x || !w || !y || (K > 1 && !ring)) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d) {
        for (int64_t b = 0; b < Bt; ++b) {
            double* r = ring ? ring + (b * D + d) * (K - 1) : NULL;
            const double xv = x[b * D + d];
            double acc = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < K; ++k) acc += w[d * K + k] * (k < K - 1 ? r[k] : xv);
            y[b * D + d] = acc * sigmoid(acc);
            for (int64_t j = 0; j + 1 < K - 1; ++j) r[j] = r[j + 1];
            if (K > 1) r[K - 2] = xv;
        }
    }
    return 0;
}
