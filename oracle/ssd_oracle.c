/*
 * ssd_oracle.c -- fp64 CPU oracle for the Mamba-2 SSD selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * What it computes (the plain sequential recurrence, one (batch, head) pair
 * at a time, every quantity in double precision):
 *
 *   dt_t  = clamp(softplus(dt_raw_t + dt_bias_h), dt_min, dt_max)
 *           (softplus optional; clamp bounds default to (0, +inf) = no clamp)
 *   h_t   = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t      (P x N)
 *   y_t   = h_t . C_t + D_h * x_t                                     (P)
 *
 * with B_t, C_t the rows of group g(h) = floor(h / (H / G)), h_{-1} the
 * initial state (or zero), and the state set to zero before any token t > 0
 * whose seq_idx differs from token t-1's.
 *
 * Sources (the pages that define the operation):
 *  - RL-Kernel RFC "Nemotron-3-Nano-30B-A3B", section 1, operator family 1:
 *    the Mamba-2 layer is a linear recurrence, computed as a chunked parallel
 *    scan in training and as a per-token recurrent state update in decode;
 *    operator family 2: a fixed-size FP32 SSM state per sequence.
 *  - same RFC, section 3, Figure 2, box [F2]: softplus(dt + dt_bias),
 *    dt_limit, A = -exp(A_log) feed the SSD scan.
 *  - "Nemotron 3 Nano - JAX Implementation", Key Components, item 1
 *    (Mamba 2 blocks): selective scan (SSD) with a D skip connection and
 *    groups of B/C shared by several heads, like GQA (Configuration,
 *    mamba_ngroups).
 *  - same RFC, section 2, "Reference-implementation hazards": the naive SSD
 *    path is checked by allclose against an FP64 re-run; section 7,
 *    "Oracles": never test a kernel against an oracle that shares its code.
 *
 * Layouts (row-major, contiguous):
 *   x (b,L,H,P)  dt_raw (b,L,H)  B,C (b,L,G,N)  y (b,L,H,P)
 *   h_init, h_final (b,H,P,N)  seq_idx (b,L) int32  dt_bias, A, D (H)
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* log(1 + e^v) evaluated without overflow: max(v,0) + log1p(e^{-|v|}). */
static double oracle_softplus(double v) {
    double m = v > 0.0 ? v : 0.0;
    return m + log1p(exp(-fabs(v)));
}

static double oracle_dt(double raw, double bias, int softplus, double dt_min,
                        double dt_max) {
    double v = raw + bias;
    if (softplus) v = oracle_softplus(v);
    if (v < dt_min) v = dt_min;
    if (v > dt_max) v = dt_max;
    return v;
}

/* One recurrence step for one (batch, head): updates s (P x N) in place and
 * writes y (P).  xt (P), bt (N), ct (N). */
static void oracle_token(int64_t P, int64_t N, double dt, double A, double Dh,
                         const double* xt, const double* bt, const double* ct,
                         double* s, double* yt) {
    double decay = exp(dt * A);
    for (int64_t p = 0; p < P; ++p) {
        double* row = s + p * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            row[n] = decay * row[n] + dt * xt[p] * bt[n];
            acc += row[n] * ct[n];
        }
        yt[p] = acc + Dh * xt[p];
    }
}

int oracle_ssd_scan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                    int64_t G, const double* x, const double* dt_raw,
                    const double* dt_bias, int dt_softplus, double dt_min,
                    double dt_max, const double* A, const double* B,
                    const double* C, const double* D, const double* h_init,
                    const int32_t* seq_idx, double* y, double* h_final,
                    int nthreads) {
    if (batch < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return 1;
    if (H % G != 0) return 2;
    if (!x || !dt_raw || !A || !B || !C || !y) return 3;
    const int64_t heads_per_group = H / G;
    const int64_t tasks = batch * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < tasks; ++task) {
        const int64_t b = task / H, h = task % H;
        const int64_t g = h / heads_per_group;
        double* s = (double*)malloc(sizeof(double) * (size_t)(P * N));
        double* yt = (double*)malloc(sizeof(double) * (size_t)P);
        if (!s || !yt) {
            failed = 1;
            free(s); free(yt);
            continue;
        }
        if (h_init)
            memcpy(s, h_init + (b * H + h) * P * N, sizeof(double) * (size_t)(P * N));
        else
            memset(s, 0, sizeof(double) * (size_t)(P * N));
        const double bias = dt_bias ? dt_bias[h] : 0.0;
        const double Dh = D ? D[h] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            if (seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1])
                memset(s, 0, sizeof(double) * (size_t)(P * N));
            const double dt = oracle_dt(dt_raw[(b * L + t) * H + h], bias,
                                        dt_softplus, dt_min, dt_max);
            const double* xrow = x + ((b * L + t) * H + h) * P;
            const double* brow = B + ((b * L + t) * G + g) * N;
            const double* crow = C + ((b * L + t) * G + g) * N;
            oracle_token(P, N, dt, A[h], Dh, xrow, brow, crow, s, yt);
            memcpy(y + ((b * L + t) * H + h) * P, yt, sizeof(double) * (size_t)P);
        }
        if (h_final)
            memcpy(h_final + (b * H + h) * P * N, s, sizeof(double) * (size_t)(P * N));
        free(s); free(yt);
    }
    return failed ? 4 : 0;
}

/* One decode token per sequence: state (b,H,P,N) updated in place,
 * x (b,H,P), dt_raw (b,H), B, C (b,G,N), y (b,H,P). */
int oracle_ssd_step(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                    double* state, const double* x, const double* dt_raw,
                    const double* dt_bias, int dt_softplus, double dt_min,
                    double dt_max, const double* A, const double* B,
                    const double* C, const double* D, double* y) {
    if (batch < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return 1;
    if (H % G != 0) return 2;
    if (!state || !x || !dt_raw || !A || !B || !C || !y) return 3;
    const int64_t heads_per_group = H / G;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / heads_per_group;
            const double dt = oracle_dt(dt_raw[b * H + h], dt_bias ? dt_bias[h] : 0.0,
                                        dt_softplus, dt_min, dt_max);
            oracle_token(P, N, dt, A[h], D ? D[h] : 0.0, x + (b * H + h) * P,
                         B + (b * G + g) * N, C + (b * G + g) * N,
                         state + (b * H + h) * P * N, y + (b * H + h) * P);
        }
    }
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
