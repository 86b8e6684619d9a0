/*
 * oracle.c -- CPU reference for the Mamba-1 (S6) block core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg do.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * It is the plain definition written out: fp64 loops, one (batch, channel)
 * column at a time, time in order, no blocking and no reordering.  Inputs are
 * the fp32 tensors the GPU also receives, promoted to fp64.  Columns are
 * independent, so OpenMP splits the work over them only and the result is
 * bitwise identical for every thread count.
 *
 * Source of every formula: the pages of the npm package
 * "@seanhogg/builderforce-memory-engine", in particular the diff
 * 2026.7.12 -> 2026.9.27, file src/training/mamba1_cpu.ts, function
 * mamba1CpuForward (steps 4, 5, 8 and 9), and the diff 2026.7.14 -> 2026.9.28,
 * file src/training/cpu_ops.ts (silu, softplus).  Layouts are the ones that
 * file's header lists: activations (M, D) with M = batch * seqLen and row
 * r = b * seqLen + t, B and C (M, N), A_log (D, N), wConv (D, K),
 * hCache (B, L, D, N).
 *
 * Readings taken where the pages leave a step open:
 *   - ZOH input term: the pages compute ((aBar - 1) / A) * B.  The oracle
 *     evaluates the same quantity as expm1(dv * A) / A * B, which has no
 *     cancellation when dv * A is close to zero.
 *   - EULER input term dv * B is the alternative discretisation; the caller
 *     chooses the mode, nothing defaults.
 *   - The optional initial state h0 and the single-token step function are
 *     extensions: the step applies the same per-step update with a carried
 *     state, the conv window taken from the last K-1 inputs (oldest first).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DISC_ZOH 0
#define ORACLE_DISC_EULER 1
#define ORACLE_MAX_N 64
#define ORACLE_MAX_K 64

/* Clamp bounds on A_log (mamba1_cpu.ts, A_LOG_CLAMP_LO / A_LOG_CLAMP_HI). */
static const double A_LOG_LO = -10.0;
static const double A_LOG_HI = 5.0;

/* SiLU(v) = v * sigmoid(v)   (cpu_ops.ts, silu). */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/* Stable softplus max(v,0) + log1p(exp(-|v|))   (cpu_ops.ts, softplus). */
static double softplus(double v) { return fmax(v, 0.0) + log1p(exp(-fabs(v))); }

/* Continuous A = -exp(clamp(A_log, LO, HI))   (mamba1CpuForward, step 8). */
static double a_cont(double a_log) {
    double c = a_log;
    if (c < A_LOG_LO) c = A_LOG_LO;
    if (c > A_LOG_HI) c = A_LOG_HI;
    return -exp(c);
}

/* Input coefficient bBar for one state: ZOH ((aBar-1)/A)*B or EULER dv*B. */
static double b_bar(int disc, double dv, double A, double Bv) {
    if (disc == ORACLE_DISC_ZOH) return expm1(dv * A) / A * Bv;
    return dv * Bv;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Step 4 + 5: causal depthwise conv1d, then SiLU.
 *   c[b,t,d] = bConv[d] + sum_{k=0}^{K-1} [t >= k] wConv[d*K+k] * x[b, t-k, d]
 * Tap k = 0 multiplies the current step; rows before the start of a batch
 * contribute nothing.                                                       */
static double conv_at(const float* x, const float* w, const float* bias,
                      int64_t L, int64_t D, int64_t K, int64_t b, int64_t t, int64_t d) {
    double acc = bias ? (double)bias[d] : 0.0;
    for (int64_t k = 0; k < K; k++) {
        if (t >= k) acc += (double)w[d * K + k] * (double)x[(b * L + t - k) * D + d];
    }
    return acc;
}

int oracle_conv1d_silu(int64_t B, int64_t L, int64_t D, int64_t K,
                       const float* x, const float* w, const float* bias,
                       double* u, int nthreads) {
    if (B < 0 || L < 0 || D < 0 || K < 1 || K > ORACLE_MAX_K) return -1;
    if (!x || !w || !u) return -1;
    int nt = set_threads(nthreads);
    int64_t cols = B * D;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t c = 0; c < cols; c++) {
        int64_t b = c / D, d = c % D;
        for (int64_t t = 0; t < L; t++)
            u[(b * L + t) * D + d] = silu(conv_at(x, w, bias, L, D, K, b, t, d));
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 8 + 9 for one (b, d) column: the selective scan and the gate.
 *   dv  = softplus(delta[r, d])
 *   A_n = -exp(clamp(A_log[d, n]))
 *   aBar = exp(dv * A_n);  bBar = ZOH or EULER term times B[r, n]
 *   h_n  = aBar * h_n + bBar * u[r, d]        (h_n = h0 or 0 before t = 0)
 *   y    = D_vec[d] * u + sum_n C[r, n] * h_n
 *   out  = y * silu(z[r, d])                  (ungated when z is absent)
 * hCache holds h after the update of step t.                                */
typedef struct {
    int64_t B, L, D, N;
    int disc;
    const float *delta, *A_log, *Bm, *Cm, *Dv, *z, *h0;
} scan_args;

static void scan_column(const scan_args* a, int64_t b, int64_t d, const double* u,
                        double* y, int64_t y_stride,
                        double* hc, int64_t hc_stride, double* hl) {
    const int64_t L = a->L, D = a->D, N = a->N;
    double A[ORACLE_MAX_N], h[ORACLE_MAX_N];
    for (int64_t n = 0; n < N; n++) {
        A[n] = a_cont((double)a->A_log[d * N + n]);
        h[n] = a->h0 ? (double)a->h0[(b * D + d) * N + n] : 0.0;
    }
    const double Dd = a->Dv ? (double)a->Dv[d] : 0.0;
    for (int64_t t = 0; t < L; t++) {
        const int64_t r = b * L + t;
        const double dv = softplus((double)a->delta[r * D + d]);
        const double uv = u[t];
        double acc = Dd * uv;
        for (int64_t n = 0; n < N; n++) {
            const double ab = exp(dv * A[n]);
            const double bb = b_bar(a->disc, dv, A[n], (double)a->Bm[r * N + n]);
            h[n] = ab * h[n] + bb * uv;
            if (hc) hc[t * hc_stride + n] = h[n];
            acc += (double)a->Cm[r * N + n] * h[n];
        }
        y[t * y_stride] = a->z ? acc * silu((double)a->z[r * D + d]) : acc;
    }
    if (hl)
        for (int64_t n = 0; n < N; n++) hl[n] = h[n];
}

/* Output layouts.  Without a column list: y (B*L, D), h_cache (B, L, D, N),
 * h_last (B, D, N).  With a column list (entries b*D + d): y (ncols, L),
 * h_cache (ncols, L, N), h_last (ncols, N).                                 */
static int scan_driver(const scan_args* a, int conv, const float* src,
                       const float* w, const float* bias, int64_t K,
                       const int64_t* cols, int64_t ncols,
                       double* y, double* h_cache, double* h_last, int nthreads) {
    const int64_t L = a->L, D = a->D, N = a->N;
    if (a->B < 0 || L < 0 || D < 0 || N < 1 || N > ORACLE_MAX_N) return -1;
    if (a->disc != ORACLE_DISC_ZOH && a->disc != ORACLE_DISC_EULER) return -1;
    if (!src || !a->delta || !a->A_log || !a->Bm || !a->Cm || !y) return -1;
    if (conv && (!w || K < 1 || K > ORACLE_MAX_K)) return -1;
    const int64_t total = cols ? ncols : a->B * D;
    for (int64_t i = 0; cols && i < ncols; i++)
        if (cols[i] < 0 || cols[i] >= a->B * D) return -1;
    int nt = set_threads(nthreads);
    int err = 0;
#pragma omp parallel num_threads(nt)
    {
        double* u = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        if (!u) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < total; i++) {
            if (!u) continue;
            const int64_t c = cols ? cols[i] : i;
            const int64_t b = c / D, d = c % D;
            for (int64_t t = 0; t < L; t++)
                u[t] = conv ? silu(conv_at(src, w, bias, L, D, K, b, t, d))
                            : (double)src[(b * L + t) * D + d];
            double *yp, *hcp = NULL, *hlp = NULL;
            int64_t ys, hcs = 0;
            if (cols) {
                yp = y + i * L; ys = 1;
                if (h_cache) { hcp = h_cache + i * L * N; hcs = N; }
                if (h_last) hlp = h_last + i * N;
            } else {
                yp = y + b * L * D + d; ys = D;
                if (h_cache) { hcp = h_cache + (b * L * D + d) * N; hcs = D * N; }
                if (h_last) hlp = h_last + (b * D + d) * N;
            }
            scan_column(a, b, d, u, yp, ys, hcp, hcs, hlp);
        }
        free(u);
    }
    return err;
}

/* Selective scan on a given u (the SiLU output). */
int oracle_selective_scan(int64_t B, int64_t L, int64_t D, int64_t N, int disc,
                          const float* u, const float* delta, const float* A_log,
                          const float* Bm, const float* Cm, const float* Dv,
                          const float* z, const float* h0,
                          const int64_t* cols, int64_t ncols,
                          double* y, double* h_cache, double* h_last, int nthreads) {
    scan_args a = {B, L, D, N, disc, delta, A_log, Bm, Cm, Dv, z, h0};
    return scan_driver(&a, 0, u, NULL, NULL, 0, cols, ncols, y, h_cache, h_last, nthreads);
}

/* Conv1d + SiLU feeding the scan, from the raw conv input x. */
int oracle_mamba1_core(int64_t B, int64_t L, int64_t D, int64_t N, int64_t K, int disc,
                       const float* x, const float* w_conv, const float* b_conv,
                       const float* delta, const float* A_log,
                       const float* Bm, const float* Cm, const float* Dv,
                       const float* z, const float* h0,
                       const int64_t* cols, int64_t ncols,
                       double* y, double* h_cache, double* h_last, int nthreads) {
    scan_args a = {B, L, D, N, disc, delta, A_log, Bm, Cm, Dv, z, h0};
    return scan_driver(&a, 1, x, w_conv, b_conv, K, cols, ncols, y, h_cache, h_last, nthreads);
}

/* ------------------------------------------------------------------------ */
/* One single-token recurrent step with carried state.
 *   window: x_{t-k} = conv_state[K-1-k] for k >= 1 (oldest first), x_t = x
 *   c = bConv + sum_k wConv[d,k] * x_{t-k};  u = silu(c)
 *   then the step-8/9 update of one time step on the carried h.
 *   conv_state' = (conv_state[1..K-2], x)
 * Layouts without a column list: x, z, delta (B, D); B, C (B, N);
 * conv_state (B, K-1, D); h (B, D, N); y (B, D).  With a column list
 * (entries b*D + d) the state and outputs are compact: conv_state (ncols,
 * K-1), h (ncols, N), y (ncols); x, z, delta, B, C keep their full layout. */
int oracle_selective_step(int64_t B, int64_t D, int64_t N, int64_t K, int disc,
                          const float* x, const float* z, const float* delta,
                          const float* A_log, const float* Bm, const float* Cm,
                          const float* Dv, const float* w_conv, const float* b_conv,
                          const double* conv_state_in, const double* h_in,
                          const int64_t* cols, int64_t ncols,
                          double* y, double* conv_state_out, double* h_out, int nthreads) {
    if (B < 0 || D < 0 || N < 1 || N > ORACLE_MAX_N || K < 1 || K > ORACLE_MAX_K) return -1;
    if (disc != ORACLE_DISC_ZOH && disc != ORACLE_DISC_EULER) return -1;
    if (!x || !delta || !A_log || !Bm || !Cm || !w_conv || !h_in || !y || !h_out) return -1;
    if (K > 1 && (!conv_state_in || !conv_state_out)) return -1;
    const int64_t total = cols ? ncols : B * D;
    for (int64_t i = 0; cols && i < ncols; i++)
        if (cols[i] < 0 || cols[i] >= B * D) return -1;
    const int64_t S = K - 1;
    int nt = set_threads(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < total; i++) {
        const int64_t c = cols ? cols[i] : i;
        const int64_t b = c / D, d = c % D;
        double win[ORACLE_MAX_K];
        for (int64_t j = 0; j < S; j++)
            win[j] = cols ? conv_state_in[i * S + j] : conv_state_in[(b * S + j) * D + d];
        const double xv = (double)x[b * D + d];
        double acc = b_conv ? (double)b_conv[d] : 0.0;
        acc += (double)w_conv[d * K + 0] * xv;
        for (int64_t k = 1; k < K; k++) acc += (double)w_conv[d * K + k] * win[S - k];
        const double uv = silu(acc);
        const double dv = softplus((double)delta[b * D + d]);
        double yv = (Dv ? (double)Dv[d] : 0.0) * uv;
        for (int64_t n = 0; n < N; n++) {
            const double A = a_cont((double)A_log[d * N + n]);
            const double ab = exp(dv * A);
            const double bb = b_bar(disc, dv, A, (double)Bm[b * N + n]);
            const int64_t hi = cols ? i * N + n : (b * D + d) * N + n;
            const double hv = ab * h_in[hi] + bb * uv;
            h_out[hi] = hv;
            yv += (double)Cm[b * N + n] * hv;
        }
        y[cols ? i : b * D + d] = z ? yv * silu((double)z[b * D + d]) : yv;
        for (int64_t j = 0; j < S; j++) {
            const double nv = (j + 1 < S) ? win[j + 1] : xv;
            if (cols) conv_state_out[i * S + j] = nv;
            else conv_state_out[(b * S + j) * D + d] = nv;
        }
    }
    return 0;
}

int oracle_abi_version(void) { return 1; }
