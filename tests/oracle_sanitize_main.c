/*
 * Host-sanitizer driver for the oracle (test infrastructure): calls every
 * entry point of oracle.c on small ragged shapes, with and without the
 * optional inputs, so that AddressSanitizer and UndefinedBehaviorSanitizer see
 * every loop and index of the oracle.  Built and run by
 * tests/test_oracle_sanitize.py as  gcc -fsanitize=address,undefined
 * oracle/oracle.c tests/oracle_sanitize_main.c.  Exits non-zero on a rejected
 * call or a non-finite result.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_softplus(double v);
double oracle_silu(double z);
void oracle_zoh(double delta, double a, double *abar, double *bcoef);
int oracle_selective_scan_fwd(const double *x, const double *dt, const double *dt_bias,
                              const double *A, const double *Bm, const double *Cm,
                              const double *Dskip, const double *z, const double *h0, double *y,
                              double *h_last, int64_t B, int64_t D, int64_t L, int64_t N,
                              int nthreads);
int oracle_conv1d_silu(const double *x, const double *w, const double *bias, double *out,
                       int64_t B, int64_t D, int64_t L, int64_t K, int apply_silu);
int oracle_conv1d_update(double *state, const double *x, const double *w, const double *bias,
                         double *out, int64_t B, int64_t D, int64_t K);
int oracle_selective_scan_bwd(const double *x, const double *dt, const double *dt_bias,
                              const double *A, const double *Bm, const double *Cm,
                              const double *Dskip, const double *z, const double *h0,
                              const double *dout, const double *dh_last, double *dx, double *ddt,
                              double *dz, double *dA, double *dD, double *ddt_bias, double *dB,
                              double *dC, double *dh0, int64_t B, int64_t D, int64_t L, int64_t N);
int oracle_state_update(double *h, const double *x, const double *dt, const double *dt_bias,
                        const double *A, const double *Bm, const double *Cm, const double *Dskip,
                        const double *z, double *y, int64_t B, int64_t D, int64_t N);
int oracle_ssd_scan_fwd(const double *x, const double *dt, const double *dt_bias,
                        const double *A, const double *Bm, const double *Cm, const double *Dskip,
                        const double *z, const double *h0, double *y, double *h_last, int64_t B,
                        int64_t L, int64_t H, int64_t P, int64_t G, int64_t N);

static unsigned rng_state = 12345u;
static double rnd(void)
{
    rng_state = rng_state * 1103515245u + 12345u;
    return ((double)((rng_state >> 8) & 0xffff) / 65536.0) * 2.0 - 1.0;
}
/* exactly-sized heap buffer (so a one-past-the-end access is caught) */
static double *buf(size_t n)
{
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    if (!p)
        exit(3);
    for (size_t i = 0; i < n; ++i)
        p[i] = rnd();
    return p;
}
static int finite_all(const double *p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i]))
            return 0;
    return 1;
}
#define CHECK(cond, what)                                                                     \
    do {                                                                                      \
        if (!(cond)) {                                                                        \
            fprintf(stderr, "FAIL: %s\n", what);                                              \
            return 1;                                                                         \
        }                                                                                     \
    } while (0)

int main(void)
{
    const int64_t B = 2, D = 3, L = 7, N = 5, K = 4;
    double *x = buf(B * D * L), *dt = buf(B * D * L), *z = buf(B * D * L), *A = buf(D * N);
    double *Bm = buf(B * L * N), *Cm = buf(B * L * N), *bias = buf(D), *Dv = buf(D);
    double *h0 = buf(B * D * N), *y = buf(B * D * L), *hl = buf(B * D * N);
    for (int64_t i = 0; i < D * N; ++i)
        A[i] = -fabs(A[i]) - 0.1;
    A[1] = 0.0;
    for (int opt = 0; opt < 2; ++opt) {
        const int full = opt == 0;
        CHECK(oracle_selective_scan_fwd(x, dt, full ? bias : NULL, A, Bm, Cm, full ? Dv : NULL,
                                        full ? z : NULL, full ? h0 : NULL, y,
                                        full ? hl : NULL, B, D, L, N, 1 + 2 * full) == 0,
              "scan");
        CHECK(finite_all(y, B * D * L), "scan y");
    }
    double *w = buf(D * K), *cb = buf(D), *co = buf(B * D * L);
    CHECK(oracle_conv1d_silu(x, w, cb, co, B, D, L, K, 1) == 0 && finite_all(co, B * D * L), "conv");
    CHECK(oracle_conv1d_silu(x, w, NULL, co, B, D, L, 1, 0) == 0, "conv K=1");
    double *st = buf(B * D * (K - 1)), *xo = buf(B * D), *uo = buf(B * D);
    CHECK(oracle_conv1d_update(st, xo, w, cb, uo, B, D, K) == 0 && finite_all(uo, B * D), "conv update");
    CHECK(oracle_conv1d_update(NULL, xo, w, NULL, uo, B, D, 1) == 0, "conv update K=1");
    double *h = buf(B * D * N), *yd = buf(B * D);
    CHECK(oracle_state_update(h, xo, xo, bias, A, Bm, Cm, Dv, xo, yd, B, D, N) == 0 &&
              finite_all(yd, B * D), "state update");
    double *dout = buf(B * D * L), *dhl = buf(B * D * N), *dx = buf(B * D * L), *ddt = buf(B * D * L);
    double *dz = buf(B * D * L), *dA = buf(D * N), *dD = buf(D), *db = buf(D), *dB = buf(B * L * N);
    double *dC = buf(B * L * N), *dh0 = buf(B * D * N);
    CHECK(oracle_selective_scan_bwd(x, dt, bias, A, Bm, Cm, Dv, z, h0, dout, dhl, dx, ddt, dz, dA,
                                    dD, db, dB, dC, dh0, B, D, L, N) == 0 &&
              finite_all(dA, D * N) && finite_all(dB, B * L * N), "backward");
    CHECK(oracle_selective_scan_bwd(x, dt, NULL, A, Bm, Cm, NULL, NULL, NULL, dout, NULL, dx, ddt,
                                    NULL, dA, dD, db, dB, dC, NULL, B, D, L, N) == 0, "backward, no options");
    const int64_t H = 4, P = 3, G = 2, Ns = 6;
    double *x2 = buf(B * L * H * P), *dt2 = buf(B * L * H), *A2 = buf(H), *B2 = buf(B * L * G * Ns);
    double *C2 = buf(B * L * G * Ns), *z2 = buf(B * L * H * P), *hh0 = buf(B * H * P * Ns);
    double *y2 = buf(B * L * H * P), *hh = buf(B * H * P * Ns), *bias2 = buf(H), *Dv2 = buf(H);
    for (int64_t i = 0; i < H; ++i)
        A2[i] = -fabs(A2[i]);
    CHECK(oracle_ssd_scan_fwd(x2, dt2, bias2, A2, B2, C2, Dv2, z2, hh0, y2, hh, B, L, H, P, G, Ns) == 0 &&
              finite_all(y2, B * L * H * P) && finite_all(hh, B * H * P * Ns), "ssd");
    CHECK(oracle_ssd_scan_fwd(x2, dt2, NULL, A2, B2, C2, NULL, NULL, NULL, y2, NULL, B, L, H, P, G, Ns) == 0,
          "ssd, no options");
    CHECK(oracle_ssd_scan_fwd(x2, dt2, NULL, A2, B2, C2, NULL, NULL, NULL, y2, NULL, B, L, H, P, 3, Ns) == -1,
          "ssd rejects H % G != 0");
    double ab, bc;
    oracle_zoh(0.5, 0.0, &ab, &bc);
    CHECK(ab == 1.0 && bc == 0.5, "zoh at A = 0");
    CHECK(isfinite(oracle_softplus(800.0)) && isfinite(oracle_silu(-800.0)), "softplus / silu range");
    printf("oracle sanitize driver: ok\n");
    /* every buffer is released so that LeakSanitizer reports only the oracle's own leaks */
    double *all[] = {x, dt, z, A, Bm, Cm, bias, Dv, h0, y, hl, w, cb, co, st, xo, uo, h, yd, dout,
                     dhl, dx, ddt, dz, dA, dD, db, dB, dC, dh0, x2, dt2, A2, B2, C2, z2, hh0, y2, hh,
                     bias2, Dv2};
    for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i)
        free(all[i]);
    return 0;
}
