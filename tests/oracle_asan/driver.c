/* Runs every entry point of the C oracle (oracle/ssm_oracle.c, oracle/conv_oracle.c)
 * on small seeded inputs, each buffer allocated at exactly the size the entry point
 * may touch, so that an AddressSanitizer / UndefinedBehaviorSanitizer build reports
 * any out-of-bounds access, use of freed memory or undefined arithmetic.  It also
 * checks two invariants the oracle guarantees: stepping token by token equals the
 * forward bit for bit (scan and conv), and a repeated call is bitwise repeatable.
 * Test infrastructure only (built and run by tests/test_oracle_asan.py). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_fwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *, const double *,
               const double *, const double *, const double *, const double *, const double *,
               const double *, double *, double *, double *);
int oracle_step(int64_t, int64_t, int64_t, double *, const double *, const double *, const double *,
                const double *, const double *, const double *, const double *, const double *, double *);
int oracle_bwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *, const double *,
               const double *, const double *, const double *, const double *, const double *,
               const double *, const double *, double *, double *, double *, double *, double *,
               double *, double *, double *, double *, double *);
int oracle_conv_fwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *, const double *,
                    const double *, double *, double *, double *);
int oracle_conv_bwd(int64_t, int64_t, int64_t, int64_t, const double *, const double *, const double *,
                    const double *, const double *, double *, double *, double *, double *);
int oracle_conv_step(int64_t, int64_t, int64_t, double *, const double *, const double *, const double *,
                     double *);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double uni(void) { /* splitmix64 -> [-1, 1) */
    uint64_t z = (rng += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static double *rnd(size_t n, double scale) {
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = scale * uni();
    return p;
}
static double *zeros(size_t n) { return (double *)calloc(n ? n : 1, sizeof(double)); }
static int fails = 0;
#define CHECK(cond, what)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            fprintf(stderr, "FAIL: %s\n", what);            \
            ++fails;                                        \
        }                                                   \
    } while (0)

static void scan_case(int64_t Bt, int64_t L, int64_t D, int64_t N, int gate, int with_h0, int with_opt) {
    const size_t btd = (size_t)(Bt * L * D), btn = (size_t)(Bt * L * N), bdn = (size_t)(Bt * D * N);
    double *x = rnd(btd, 1.0), *dt = rnd(btd, 2.0), *B = rnd(btn, 1.0), *C = rnd(btn, 1.0);
    double *z = gate ? rnd(btd, 2.0) : NULL, *dy = rnd(btd, 1.0);
    double *A_log = rnd((size_t)(D * N), 1.0), *Dp = with_opt ? rnd((size_t)D, 1.0) : NULL;
    double *bias = with_opt ? rnd((size_t)D, 1.0) : NULL, *h0 = with_h0 ? rnd(bdn, 0.5) : NULL;
    double *y = zeros(btd), *y2 = zeros(btd), *hl = zeros(bdn), *del = zeros(btd);
    CHECK(oracle_fwd(Bt, L, D, N, x, dt, B, C, z, A_log, Dp, bias, h0, y, hl, del) == 0, "fwd rc");
    CHECK(oracle_fwd(Bt, L, D, N, x, dt, B, C, z, A_log, Dp, bias, h0, y2, NULL, NULL) == 0, "fwd rc 2");
    CHECK(memcmp(y, y2, btd * sizeof(double)) == 0, "fwd repeatable");
    /* step chain from the same start equals the forward bit for bit */
    double *h = zeros(bdn), *xs = zeros((size_t)(Bt * D)), *ds = zeros((size_t)(Bt * D));
    double *zs = zeros((size_t)(Bt * D)), *Bs = zeros((size_t)(Bt * N)), *Cs = zeros((size_t)(Bt * N));
    double *ys = zeros((size_t)(Bt * D));
    if (h0) memcpy(h, h0, bdn * sizeof(double));
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t b = 0; b < Bt; ++b) {
            for (int64_t d = 0; d < D; ++d) {
                const size_t i = (size_t)((b * L + t) * D + d), j = (size_t)(b * D + d);
                xs[j] = x[i];
                ds[j] = dt[i];
                if (z) zs[j] = z[i];
            }
            for (int64_t n = 0; n < N; ++n) {
                Bs[b * N + n] = B[(b * L + t) * N + n];
                Cs[b * N + n] = C[(b * L + t) * N + n];
            }
        }
        CHECK(oracle_step(Bt, D, N, h, xs, ds, Bs, Cs, z ? zs : NULL, A_log, Dp, bias, ys) == 0, "step rc");
        for (int64_t b = 0; b < Bt; ++b)
            for (int64_t d = 0; d < D; ++d)
                CHECK(ys[b * D + d] == y[(b * L + t) * D + d], "step == fwd");
    }
    CHECK(L == 0 || memcmp(h, hl, bdn * sizeof(double)) == 0, "step state == h_last");
    double *dx = zeros(btd), *ddt = zeros(btd), *dB = zeros(btn), *dC = zeros(btn), *dz = zeros(btd);
    double *dA = zeros((size_t)(D * N)), *dD = zeros((size_t)D), *ddb = zeros((size_t)D), *dh0 = zeros(bdn);
    double *ddel = zeros(btd), *dx2 = zeros(btd);
    CHECK(oracle_bwd(Bt, L, D, N, x, dt, B, C, z, A_log, Dp, bias, h0, dy, dx, ddt, dB, dC, z ? dz : NULL, dA,
                     dD, ddb, dh0, ddel) == 0, "bwd rc");
    CHECK(oracle_bwd(Bt, L, D, N, x, dt, B, C, z, A_log, Dp, bias, h0, dy, dx2, ddt, dB, dC, z ? dz : NULL,
                     dA, dD, ddb, NULL, NULL) == 0, "bwd rc 2");
    CHECK(memcmp(dx, dx2, btd * sizeof(double)) == 0, "bwd repeatable");
    double *bufs[] = {x, dt, B, C, z, dy, A_log, Dp, bias, h0, y, y2, hl, del, h, xs, ds, zs, Bs, Cs, ys,
                      dx, ddt, dB, dC, dz, dA, dD, ddb, dh0, ddel, dx2};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) free(bufs[i]);
}

static void conv_case(int64_t Bt, int64_t L, int64_t D, int64_t K, int with_ring, int with_bias) {
    const size_t btd = (size_t)(Bt * L * D), ring = (size_t)(Bt * D * (K - 1));
    double *x = rnd(btd, 1.0), *w = rnd((size_t)(D * K), 0.5), *b = with_bias ? rnd((size_t)D, 0.3) : NULL;
    double *s0 = (with_ring && K > 1) ? rnd(ring, 1.0) : NULL, *dy = rnd(btd, 1.0);
    double *y = zeros(btd), *sl = zeros(ring), *pre = zeros(btd);
    CHECK(oracle_conv_fwd(Bt, L, D, K, x, w, b, s0, y, K > 1 ? sl : NULL, pre) == 0, "conv fwd rc");
    double *r = zeros(ring), *xs = zeros((size_t)(Bt * D)), *ys = zeros((size_t)(Bt * D));
    if (s0) memcpy(r, s0, ring * sizeof(double));
    for (int64_t t = 0; t < L; ++t) {
        for (int64_t bb = 0; bb < Bt; ++bb)
            for (int64_t d = 0; d < D; ++d) xs[bb * D + d] = x[(bb * L + t) * D + d];
        CHECK(oracle_conv_step(Bt, D, K, K > 1 ? r : NULL, xs, w, b, ys) == 0, "conv step rc");
        for (int64_t bb = 0; bb < Bt; ++bb)
            for (int64_t d = 0; d < D; ++d) CHECK(ys[bb * D + d] == y[(bb * L + t) * D + d], "conv step == fwd");
    }
    CHECK(K == 1 || L == 0 || memcmp(r, sl, ring * sizeof(double)) == 0, "conv ring == s_last");
    double *dx = zeros(btd), *dw = zeros((size_t)(D * K)), *db = zeros((size_t)D), *ds0 = zeros(ring);
    CHECK(oracle_conv_bwd(Bt, L, D, K, x, w, b, s0, dy, dx, dw, db, K > 1 ? ds0 : NULL) == 0, "conv bwd rc");
    double *bufs[] = {x, w, b, s0, dy, y, sl, pre, r, xs, ys, dx, dw, db, ds0};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) free(bufs[i]);
}

int main(void) {
    /* (batch, seqlen, channels, states), gate, h0, optional parameters */
    scan_case(2, 7, 3, 16, 1, 1, 1);
    scan_case(1, 1, 1, 1, 0, 0, 0);
    scan_case(3, 33, 5, 4, 1, 0, 1);
    scan_case(1, 0, 2, 16, 1, 1, 1);
    scan_case(2, 70, 130, 16, 1, 1, 1); /* more than one channel block in the dB/dC partials */
    for (int64_t K = 1; K <= 4; ++K) {
        conv_case(2, 9, 5, K, 1, 1);
        conv_case(1, 2, 3, K, 0, 0); /* fewer tokens than the kernel width */
        conv_case(3, 0, 4, K, 1, 1);
    }
    if (fails) {
        fprintf(stderr, "%d check(s) failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
