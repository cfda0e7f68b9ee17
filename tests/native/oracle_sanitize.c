/*
 * Driver for a host AddressSanitizer / UndefinedBehaviorSanitizer build of
 * the fp64 oracle (oracle/ssd_oracle.c): runs the scan, the decode step and
 * the gradients on small inputs that exercise every branch (packed
 * sequences, initial states, D, dt_bias, a clamp that binds, several heads
 * per group, several rows, lengths around the gradient's checkpoint stride)
 * and checks that every output is finite.  Exit status 0 on success; the
 * sanitizers abort on any invalid access or undefined operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_ssd_scan(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    const double* x, const double* dt_raw, const double* dt_bias, int softplus,
                    double dt_min, double dt_max, const double* A, const double* B,
                    const double* C, const double* D, const double* h_init,
                    const int32_t* seq_idx, double* y, double* h_final, int nthreads);
int oracle_ssd_step(int64_t b, int64_t H, int64_t P, int64_t N, int64_t G, double* state,
                    const double* x, const double* dt_raw, const double* dt_bias, int softplus,
                    double dt_min, double dt_max, const double* A, const double* B,
                    const double* C, const double* D, double* y);
int oracle_ssd_scan_bwd(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double* x, const double* dt_raw, const double* dt_bias, int softplus,
                        double dt_min, double dt_max, const double* A, const double* B,
                        const double* C, const double* D, const double* h_init,
                        const int32_t* seq_idx, const double* dy, const double* dh_final,
                        double* dx, double* ddt_raw, double* dA, double* dB, double* dC,
                        double* dD, double* ddt_bias, double* dh_init, int nthreads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(size_t n, double scale) {
    double* a = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = scale * urand();
    return a;
}
static int all_finite(const double* a, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static int run(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int packed) {
    const size_t nx = (size_t)(b * L * H * P), nd = (size_t)(b * L * H), nb = (size_t)(b * L * G * N),
                 ns = (size_t)(b * H * P * N);
    double *x = arr(nx, 1.0), *dt = arr(nd, 1.0), *B = arr(nb, 0.3), *C = arr(nb, 0.3);
    double *A = arr((size_t)H, 1.0), *D = arr((size_t)H, 1.0), *bias = arr((size_t)H, 1.0);
    for (int64_t h = 0; h < H; ++h) { A[h] = -1.0 - 4.0 * fabs(A[h]); bias[h] = -3.0 + bias[h]; }
    double *h0 = arr(ns, 0.1), *dy = arr(nx, 1.0), *dhf = arr(ns, 1.0);
    int32_t* seq = NULL;
    if (packed) {
        seq = (int32_t*)malloc((size_t)(b * L) * sizeof(int32_t));
        for (int64_t r = 0; r < b; ++r)
            for (int64_t t = 0; t < L; ++t) seq[r * L + t] = (int32_t)(3 * t / (L > 0 ? L : 1));
    }
    double *y = malloc(nx * sizeof(double)), *hf = malloc(ns * sizeof(double));
    int rc = oracle_ssd_scan(b, L, H, P, N, G, x, dt, bias, 1, 0.01, 0.5, A, B, C, D, h0, seq, y, hf, 2);
    int ok = rc == 0 && all_finite(y, nx) && all_finite(hf, ns);
    double* st = malloc(ns * sizeof(double));
    for (size_t i = 0; i < ns; ++i) st[i] = hf[i];
    double* ys = malloc((size_t)(b * H * P) * sizeof(double));
    double *xs = arr((size_t)(b * H * P), 1.0), *dts = arr((size_t)(b * H), 1.0);
    double *Bs = arr((size_t)(b * G * N), 0.3), *Cs = arr((size_t)(b * G * N), 0.3);
    rc = oracle_ssd_step(b, H, P, N, G, st, xs, dts, bias, 1, 0.0, INFINITY, A, Bs, Cs, D, ys);
    ok = ok && rc == 0 && all_finite(ys, (size_t)(b * H * P)) && all_finite(st, ns);
    free(xs); free(dts); free(Bs); free(Cs);
    double *dx = malloc(nx * sizeof(double)), *ddt = malloc(nd * sizeof(double));
    double *dA = malloc((size_t)H * sizeof(double)), *dD = malloc((size_t)H * sizeof(double));
    double *dbias = malloc((size_t)H * sizeof(double)), *dh0 = malloc(ns * sizeof(double));
    double *dB = malloc(nb * sizeof(double)), *dC = malloc(nb * sizeof(double));
    rc = oracle_ssd_scan_bwd(b, L, H, P, N, G, x, dt, bias, 1, 0.01, 0.5, A, B, C, D, h0, seq, dy, dhf,
                             dx, ddt, dA, dB, dC, dD, dbias, dh0, 2);
    ok = ok && rc == 0 && all_finite(dx, nx) && all_finite(ddt, nd) && all_finite(dB, nb) &&
         all_finite(dC, nb) && all_finite(dh0, ns) && all_finite(dA, (size_t)H) &&
         all_finite(dD, (size_t)H);
    free(x); free(dt); free(B); free(C); free(A); free(D); free(bias); free(h0); free(dy);
    free(dhf); free(seq); free(y); free(hf); free(st); free(ys); free(dx); free(ddt); free(dA);
    free(dD); free(dbias); free(dh0); free(dB); free(dC);
    if (!ok) fprintf(stderr, "case b=%lld L=%lld H=%lld P=%lld N=%lld G=%lld packed=%d failed\n",
                     (long long)b, (long long)L, (long long)H, (long long)P, (long long)N,
                     (long long)G, packed);
    return ok;
}

int main(void) {
    int ok = 1;
    ok &= run(2, 130, 4, 8, 16, 2, 1);
    ok &= run(1, 64, 2, 4, 8, 1, 0);
    ok &= run(1, 65, 2, 4, 8, 2, 1);
    ok &= run(3, 1, 2, 4, 8, 1, 0);
    ok &= run(1, 0, 2, 4, 8, 1, 0);
    printf(ok ? "oracle sanitize: ok\n" : "oracle sanitize: FAILED\n");
    return ok ? 0 : 1;
}
