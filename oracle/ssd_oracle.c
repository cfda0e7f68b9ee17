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
 *    the Mamba-2 layer's recurrence, evaluated chunk-parallel for prefill and
 *    training and one token at a time for decode; operator family 2: each
 *    sequence keeps an FP32 state of fixed size.
 *  - same RFC, section 3, Figure 2, box [F2]: softplus(dt + dt_bias),
 *    dt_limit, A = -exp(A_log) feed the SSD scan.
 *  - "Nemotron 3 Nano - JAX Implementation", Key Components, item 1
 *    (Mamba 2 blocks): selective scan (SSD) with a D skip connection and
 *    groups of B/C shared by several heads, like GQA (Configuration,
 *    mamba_ngroups).
 *  - same RFC, section 2, "Reference-implementation hazards": the naive SSD
 *    path is compared, within a tolerance, with a double-precision rerun;
 *    section 7, "Oracles": the reference a kernel is checked against must be
 *    written separately from it.
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

/* Gradients of the scan (reverse mode of the same recurrence, in the same
 * order of definitions), for a loss whose gradients with respect to y and to
 * the final state are dy (b,L,H,P) and dh_final (b,H,P,N, or NULL = 0).
 * With g_t the gradient with respect to h_t (all later uses included):
 *
 *   g_t      = dy_t (outer) C_t + [no reset at t+1] a_{t+1} g_{t+1}
 *              (+ dh_final at the last token),  a_t = exp(dt_t A)
 *   dx_t     = dt_t g_t B_t + D dy_t
 *   dB_t     = sum over the group's heads of dt_t g_t^T x_t
 *   dC_t     = sum over the group's heads of h_t^T dy_t
 *   d(dt_t)  = x_t . (g_t B_t) + [no reset at t] A a_t <g_t, h_{t-1}>
 *   dA       = sum_t [no reset at t] dt_t a_t <g_t, h_{t-1}>
 *   dD       = sum_t dy_t . x_t
 *   dh_init  = a_0 g_0
 *   d(dt_raw_t) = d(dt_t) * [dt_min <= s_t <= dt_max] * (softplus ? sigmoid(v_t) : 1),
 *              v_t = dt_raw_t + dt_bias, s_t = softplus(v_t) or v_t;
 *   d(dt_bias) = sum_t d(dt_raw_t).
 *
 * The states h_t are kept at every kCkpt-th token and recomputed forward
 * within each stretch as the reverse pass reaches it, so memory stays at
 * (L / kCkpt + kCkpt) states per (batch, head).  Sums over heads and rows are
 * taken in a fixed order after the parallel loop (deterministic).
 * Outputs (all may be NULL except dx): dx (b,L,H,P), ddt_raw (b,L,H),
 * dA, dD, ddt_bias (H), dB, dC (b,L,G,N), dh_init (b,H,P,N). */
enum { kCkpt = 64 };

int oracle_ssd_scan_bwd(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                        int64_t G, const double* x, const double* dt_raw,
                        const double* dt_bias, int dt_softplus, double dt_min,
                        double dt_max, const double* A, const double* B,
                        const double* C, const double* D, const double* h_init,
                        const int32_t* seq_idx, const double* dy, const double* dh_final,
                        double* dx, double* ddt_raw, double* dA, double* dB, double* dC,
                        double* dD, double* ddt_bias, double* dh_init, int nthreads) {
    if (batch < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return 1;
    if (H % G != 0) return 2;
    if (!x || !dt_raw || !A || !B || !C || !dy || !dx) return 3;
    const int64_t hpg = H / G;
    const int64_t tasks = batch * H;
    const int64_t PN = P * N;
    /* per-(batch, head) partials: dB, dC per head, and the per-head sums */
    double* dBh = (double*)calloc((size_t)(batch * L * H * N) + 1, sizeof(double));
    double* dCh = (double*)calloc((size_t)(batch * L * H * N) + 1, sizeof(double));
    double* sA = (double*)calloc((size_t)tasks + 1, sizeof(double));
    double* sD = (double*)calloc((size_t)tasks + 1, sizeof(double));
    double* sbias = (double*)calloc((size_t)tasks + 1, sizeof(double));
    if (!dBh || !dCh || !sA || !sD || !sbias) {
        free(dBh); free(dCh); free(sA); free(sD); free(sbias);
        return 4;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < tasks; ++task) {
        const int64_t b = task / H, h = task % H;
        const int64_t g = h / hpg;
        const int64_t nck = (L + kCkpt - 1) / kCkpt;
        /* ckpt[k]: the state before token k*kCkpt (before its reset, if any) */
        double* ckpt = (double*)malloc(sizeof(double) * (size_t)((nck + 1) * PN));
        double* hs = (double*)malloc(sizeof(double) * (size_t)((kCkpt + 1) * PN));
        double* gs = (double*)malloc(sizeof(double) * (size_t)PN);
        double* ub = (double*)malloc(sizeof(double) * (size_t)P);
        if (!ckpt || !hs || !gs || !ub) {
            failed = 1;
            free(ckpt); free(hs); free(gs); free(ub);
            continue;
        }
        const double bias = dt_bias ? dt_bias[h] : 0.0;
        const double Dh = D ? D[h] : 0.0;
        const double Ah = A[h];
        /* forward pass: checkpoints */
        double* s = ckpt;
        if (h_init) memcpy(s, h_init + (b * H + h) * PN, sizeof(double) * (size_t)PN);
        else memset(s, 0, sizeof(double) * (size_t)PN);
        for (int64_t k = 0; k < nck; ++k) {
            double* nxt = ckpt + (k + 1) * PN;
            memcpy(nxt, ckpt + k * PN, sizeof(double) * (size_t)PN);
            for (int64_t t = k * kCkpt; t < L && t < (k + 1) * kCkpt; ++t) {
                if (seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1])
                    memset(nxt, 0, sizeof(double) * (size_t)PN);
                const double dt = oracle_dt(dt_raw[(b * L + t) * H + h], bias, dt_softplus, dt_min, dt_max);
                const double a = exp(dt * Ah);
                const double* xt = x + ((b * L + t) * H + h) * P;
                const double* bt = B + ((b * L + t) * G + g) * N;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        nxt[p * N + n] = a * nxt[p * N + n] + dt * xt[p] * bt[n];
            }
        }
        /* reverse pass */
        if (dh_final) memcpy(gs, dh_final + (b * H + h) * PN, sizeof(double) * (size_t)PN);
        else memset(gs, 0, sizeof(double) * (size_t)PN);
        double accA = 0.0, accD = 0.0, accBias = 0.0;
        for (int64_t k = nck - 1; k >= 0; --k) {
            const int64_t t0 = k * kCkpt;
            const int64_t t1 = (t0 + kCkpt < L) ? t0 + kCkpt : L;
            /* hs[i] = state before token t0 + i (after no reset), hs[i+1] = h_{t0+i};
             * hs[0] is the checkpoint */
            memcpy(hs, ckpt + k * PN, sizeof(double) * (size_t)PN);
            for (int64_t t = t0; t < t1; ++t) {
                double* prev = hs + (t - t0) * PN;
                double* cur = prev + PN;
                const int reset = seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1];
                const double dt = oracle_dt(dt_raw[(b * L + t) * H + h], bias, dt_softplus, dt_min, dt_max);
                const double a = exp(dt * Ah);
                const double* xt = x + ((b * L + t) * H + h) * P;
                const double* bt = B + ((b * L + t) * G + g) * N;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        cur[p * N + n] = (reset ? 0.0 : a * prev[p * N + n]) + dt * xt[p] * bt[n];
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const double* prev = hs + (t - t0) * PN;  /* h_{t-1} before the reset test */
                const double* cur = prev + PN;            /* h_t */
                const int reset = seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1];
                const double v = dt_raw[(b * L + t) * H + h] + bias;
                const double sp = dt_softplus ? oracle_softplus(v) : v;
                const double dt = oracle_dt(dt_raw[(b * L + t) * H + h], bias, dt_softplus, dt_min, dt_max);
                const double a = exp(dt * Ah);
                const double* xt = x + ((b * L + t) * H + h) * P;
                const double* bt = B + ((b * L + t) * G + g) * N;
                const double* ct = C + ((b * L + t) * G + g) * N;
                const double* dyt = dy + ((b * L + t) * H + h) * P;
                double* dct = dCh + ((b * L + t) * H + h) * N;
                double* dbt = dBh + ((b * L + t) * H + h) * N;
                /* y_t = h_t C_t + D x_t */
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) gs[p * N + n] += dyt[p] * ct[n];
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) acc += cur[p * N + n] * dyt[p];
                    dct[n] = acc;
                }
                for (int64_t p = 0; p < P; ++p) accD += dyt[p] * xt[p];
                /* h_t = [no reset] a h_{t-1} + dt x_t B_t^T */
                double ddt = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) acc += gs[p * N + n] * bt[n];
                    ub[p] = acc;
                    dx[((b * L + t) * H + h) * P + p] = dt * acc + Dh * dyt[p];
                    ddt += xt[p] * acc;
                }
                for (int64_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < P; ++p) acc += gs[p * N + n] * xt[p];
                    dbt[n] = dt * acc;
                }
                if (!reset) {
                    double gh = 0.0;
                    for (int64_t i = 0; i < PN; ++i) gh += gs[i] * prev[i];
                    ddt += Ah * a * gh;
                    accA += dt * a * gh;
                    for (int64_t i = 0; i < PN; ++i) gs[i] *= a;
                } else {
                    memset(gs, 0, sizeof(double) * (size_t)PN);
                }
                const int pass = sp >= dt_min && sp <= dt_max;
                double draw = 0.0;
                if (pass) draw = dt_softplus ? ddt / (1.0 + exp(-v)) : ddt;
                if (ddt_raw) ddt_raw[(b * L + t) * H + h] = draw;
                accBias += draw;
            }
        }
        /* gs now holds the gradient with respect to the state before token 0 */
        if (dh_init) memcpy(dh_init + (b * H + h) * PN, gs, sizeof(double) * (size_t)PN);
        sA[task] = accA;
        sD[task] = accD;
        sbias[task] = accBias;
        free(ckpt); free(hs); free(gs); free(ub);
    }
    if (!failed) {
        for (int64_t h = 0; h < H; ++h) {
            double a = 0.0, d = 0.0, bb = 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                a += sA[b * H + h];
                d += sD[b * H + h];
                bb += sbias[b * H + h];
            }
            if (dA) dA[h] = a;
            if (dD) dD[h] = d;
            if (ddt_bias) ddt_bias[h] = bb;
        }
        for (int64_t r = 0; r < batch * L; ++r)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t n = 0; n < N; ++n) {
                    double sb = 0.0, sc = 0.0;
                    for (int64_t hh = 0; hh < hpg; ++hh) {
                        sb += dBh[(r * H + g * hpg + hh) * N + n];
                        sc += dCh[(r * H + g * hpg + hh) * N + n];
                    }
                    if (dB) dB[(r * G + g) * N + n] = sb;
                    if (dC) dC[(r * G + g) * N + n] = sc;
                }
    }
    free(dBh); free(dCh); free(sA); free(sD); free(sbias);
    return failed ? 4 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
