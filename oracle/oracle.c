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
 * mamba1CpuForward (steps 4, 5, 8 and 9) and mamba1CpuBackward (the gate,
 * the reverse-time scan adjoint, softplus, SiLU and conv1d parts), and the
 * diff 2026.7.14 -> 2026.9.28, file src/training/cpu_ops.ts (silu, softplus).  Layouts are the ones that
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

/* ------------------------------------------------------------------------ */
/* Backward pass of steps 8 + 9 (the scan and the gate), from the reverse-time
 * adjoint in the same diff's mamba1CpuBackward ("Selective scan, walked
 * backwards in time", and the gate and softplus parts around it).  Given the
 * gradient dout of the gated output:
 *   dY = dout * silu(z)                 dz = dout * y * silu'(z)   (y ungated)
 *   dD_vec[d] += dY * u                 du = dY * D_vec[d] + sum_n dh_n * bBar_n
 *   dh_n  = dY * C[r,n] + g_n           (g_n = dL/dh_t carried from step t+1)
 *   dC[r,n] += dY * h_t,n               dB[r,n] += dh_n * u * dbBar/dB
 *   g_n  <- dh_n * aBar_n               (flows to step t-1)
 *   ddv  = sum_n dh_n h_{t-1,n} A_n aBar_n + dh_n u dbBar/ddv
 *   dA_n += dh_n h_{t-1,n} dv aBar_n + dh_n u dbBar/dA
 *   ddelta = ddv * sigmoid(delta)       dA_log = dA * A inside the clamp, else 0
 *   dh0 = g after step 0
 * with, for ZOH bBar = expm1(dv A)/A * B:
 *   dbBar/dB = expm1(dv A)/A,  dbBar/ddv = aBar B,
 *   dbBar/dA = B (dv A aBar - expm1(dv A)) / A^2   (written as B dv^2 phi(dv A)
 *   with phi(x) = (x e^x - expm1(x)) / x^2, a series for small |x|, so the
 *   difference does not cancel), and for EULER bBar = dv B:
 *   dbBar/dB = dv, dbBar/ddv = B, dbBar/dA = 0.
 * The clamp boundary itself counts as outside (zero gradient), as on the pages. */
static double phi_zoh(double x) {
    if (fabs(x) < 1e-2) {
        /* sum_{k>=2} (k-1)/k! x^(k-2) */
        double term = 0.0, xp = 1.0, fact = 2.0;
        for (int k = 2; k < 12; k++) {
            term += (double)(k - 1) / fact * xp;
            xp *= x;
            fact *= (double)(k + 1);
        }
        return term;
    }
    return (x * exp(x) - expm1(x)) / (x * x);
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* d silu / dv = s (1 + v (1 - s)),  s = sigmoid(v). */
static double silu_grad(double v) {
    const double s = sigmoid(v);
    return s * (1.0 + v * (1.0 - s));
}

typedef struct {
    int64_t B, L, D, N;
    int disc;
    const float *u, *delta, *A_log, *Bm, *Cm, *Dv, *z, *h0, *dout;
} bwd_args;

/* One (b, d) column.  hs holds (L + 1) * N states (h_{-1} .. h_{L-1}).
 * Column-local outputs go straight to du, ddelta, dz, dh0; the cross-column
 * sums are written per column (dB_col, dC_col: L * N; dA_col: N; dD_col: 1)
 * and reduced afterwards in a fixed order.                                  */
static void scan_column_bwd(const bwd_args* a, int64_t b, int64_t d, double* hs, double* ys,
                            double* du, double* ddelta, double* dz, double* dh0,
                            double* dB_col, double* dC_col, double* dA_col, double* dD_col) {
    const int64_t L = a->L, D = a->D, N = a->N;
    double A[ORACLE_MAX_N], g[ORACLE_MAX_N], dA[ORACLE_MAX_N];
    for (int64_t n = 0; n < N; n++) {
        A[n] = a_cont((double)a->A_log[d * N + n]);
        hs[n] = a->h0 ? (double)a->h0[(b * D + d) * N + n] : 0.0;
        g[n] = 0.0;
        dA[n] = 0.0;
    }
    const double Dd = a->Dv ? (double)a->Dv[d] : 0.0;
    /* Forward: the states and the ungated output of every step. */
    for (int64_t t = 0; t < L; t++) {
        const int64_t r = b * L + t;
        const double dv = softplus((double)a->delta[r * D + d]);
        const double uv = (double)a->u[r * D + d];
        double yv = Dd * uv;
        for (int64_t n = 0; n < N; n++) {
            const double ab = exp(dv * A[n]);
            const double bb = b_bar(a->disc, dv, A[n], (double)a->Bm[r * N + n]);
            hs[(t + 1) * N + n] = ab * hs[t * N + n] + bb * uv;
            yv += (double)a->Cm[r * N + n] * hs[(t + 1) * N + n];
        }
        ys[t] = yv;
    }
    /* Reverse. */
    double dDsum = 0.0;
    for (int64_t t = L - 1; t >= 0; t--) {
        const int64_t r = b * L + t;
        const double dl = (double)a->delta[r * D + d];
        const double dv = softplus(dl);
        const double uv = (double)a->u[r * D + d];
        const double go = (double)a->dout[r * D + d];
        double dY = go;
        if (a->z) {
            const double zv = (double)a->z[r * D + d];
            dY = go * silu(zv);
            dz[r * D + d] = go * ys[t] * silu_grad(zv);
        }
        dDsum += dY * uv;
        double duv = dY * Dd;
        double ddv = 0.0;
        for (int64_t n = 0; n < N; n++) {
            const double Bv = (double)a->Bm[r * N + n];
            const double Cv = (double)a->Cm[r * N + n];
            const double x = dv * A[n];
            const double ab = exp(x);
            const double hprev = hs[t * N + n];
            const double hcur = hs[(t + 1) * N + n];
            dC_col[t * N + n] = dY * hcur;
            const double dh = dY * Cv + g[n];
            const double dab = dh * hprev;      /* dL/d aBar */
            const double dbb = dh * uv;         /* dL/d bBar */
            duv += dh * b_bar(a->disc, dv, A[n], Bv);
            g[n] = dh * ab;
            if (a->disc == ORACLE_DISC_ZOH) {
                ddv += dab * A[n] * ab + dbb * ab * Bv;
                dA[n] += dab * dv * ab + dbb * Bv * dv * dv * phi_zoh(x);
                dB_col[t * N + n] = dbb * expm1(x) / A[n];
            } else {
                ddv += dab * A[n] * ab + dbb * Bv;
                dA[n] += dab * dv * ab;
                dB_col[t * N + n] = dbb * dv;
            }
        }
        du[r * D + d] = duv;
        ddelta[r * D + d] = ddv * sigmoid(dl);
    }
    for (int64_t n = 0; n < N; n++) {
        const double al = (double)a->A_log[d * N + n];
        dA_col[n] = (al <= A_LOG_LO || al >= A_LOG_HI) ? 0.0 : dA[n] * A[n];
        if (dh0) dh0[(b * D + d) * N + n] = g[n];
    }
    *dD_col = dDsum;
}

/* Outputs (all fp64, dense): du, ddelta, dz (B*L, D); dA_log (D, N);
 * dB, dC (B*L, N); dD (D); dh0 (B, D, N).  dz may be NULL when z is NULL;
 * dh0 may be NULL.                                                          */
int oracle_selective_scan_backward(int64_t B, int64_t L, int64_t D, int64_t N, int disc,
                                   const float* u, const float* delta, const float* A_log,
                                   const float* Bm, const float* Cm, const float* Dv,
                                   const float* z, const float* h0, const float* dout,
                                   double* du, double* ddelta, double* dA_log, double* dB,
                                   double* dC, double* dD, double* dz, double* dh0,
                                   int nthreads) {
    if (B < 0 || L < 0 || D < 0 || N < 1 || N > ORACLE_MAX_N) return -1;
    if (disc != ORACLE_DISC_ZOH && disc != ORACLE_DISC_EULER) return -1;
    if (!u || !delta || !A_log || !Bm || !Cm || !dout) return -1;
    if (!du || !ddelta || !dA_log || !dB || !dC || !dD) return -1;
    if (z && !dz) return -1;
    bwd_args a = {B, L, D, N, disc, u, delta, A_log, Bm, Cm, Dv, z, h0, dout};
    /* The sums over d of the per-column dB, dC rows are taken in a fixed
     * order without storing every column: the channels of a batch row are
     * cut into blocks of 64, each block adds its columns in
     * channel order into a block buffer (L*N), and the blocks are added in
     * order at the end.  Bitwise identical for any thread count. */
    const int64_t BLK = 64;
    const int64_t nblk_b = D > 0 ? (D + BLK - 1) / BLK : 0;
    const int64_t nblk = B * nblk_b;
    const int64_t LN = L * N;
    double* blkB = (double*)calloc((size_t)(nblk * LN + 1), sizeof(double));
    double* blkC = (double*)calloc((size_t)(nblk * LN + 1), sizeof(double));
    double* colA = (double*)calloc((size_t)(B * D * N + 1), sizeof(double));
    double* colD = (double*)calloc((size_t)(B * D + 1), sizeof(double));
    if (!blkB || !blkC || !colA || !colD) {
        free(blkB); free(blkC); free(colA); free(colD);
        return -2;
    }
    int nt = set_threads(nthreads);
    int err = 0;
#pragma omp parallel num_threads(nt)
    {
        double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));
        double* ys = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double* cb = (double*)malloc(sizeof(double) * (size_t)(LN > 0 ? LN : 1));
        double* cc = (double*)malloc(sizeof(double) * (size_t)(LN > 0 ? LN : 1));
        if (!hs || !ys || !cb || !cc) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t k = 0; k < nblk; k++) {
            if (!hs || !ys || !cb || !cc) continue;
            const int64_t b = k / nblk_b, d0 = (k % nblk_b) * BLK;
            const int64_t d1 = d0 + BLK < D ? d0 + BLK : D;
            for (int64_t d = d0; d < d1; d++) {
                scan_column_bwd(&a, b, d, hs, ys, du, ddelta, dz, dh0, cb, cc,
                                colA + (b * D + d) * N, colD + b * D + d);
                for (int64_t i = 0; i < LN; i++) {
                    blkB[k * LN + i] += cb[i];
                    blkC[k * LN + i] += cc[i];
                }
            }
        }
        free(hs);
        free(ys);
        free(cb);
        free(cc);
    }
    if (err == 0) {
        /* dB, dC: blocks of a batch row in order; dA_log, dD: over b. */
#pragma omp parallel for schedule(static) num_threads(nt)
        for (int64_t i = 0; i < B * LN; i++) {
            const int64_t b = i / LN, tn = i % LN;
            double sb = 0.0, sc = 0.0;
            for (int64_t q = 0; q < nblk_b; q++) {
                sb += blkB[(b * nblk_b + q) * LN + tn];
                sc += blkC[(b * nblk_b + q) * LN + tn];
            }
            dB[i] = sb;
            dC[i] = sc;
        }
        for (int64_t i = 0; i < D * N; i++) {
            const int64_t d = i / N, n = i % N;
            double s = 0.0;
            for (int64_t b = 0; b < B; b++) s += colA[(b * D + d) * N + n];
            dA_log[i] = s;
        }
        for (int64_t d = 0; d < D; d++) {
            double s = 0.0;
            for (int64_t b = 0; b < B; b++) s += colD[b * D + d];
            dD[d] = s;
        }
    }
    free(blkB); free(blkC); free(colA); free(colD);
    return err;
}

/* Backward of steps 4 + 5 (the same diff's mamba1CpuBackward, "SiLU" and
 * "Depthwise causal conv1d"): with c the conv output and dc = du * silu'(c),
 *   dx[b, t-k, d] += dc[b,t,d] * wConv[d,k]   (t >= k)
 *   dwConv[d,k]   += dc[b,t,d] * x[b, t-k, d]
 *   dbConv[d]     += dc[b,t,d]
 * du is the total gradient reaching u.  Outputs fp64: dx (B*L, D),
 * dw (D, K), db (D).                                                        */
int oracle_conv1d_silu_backward(int64_t B, int64_t L, int64_t D, int64_t K,
                                const float* x, const float* w, const float* bias,
                                const float* du, double* dx, double* dw, double* db,
                                int nthreads) {
    if (B < 0 || L < 0 || D < 0 || K < 1 || K > ORACLE_MAX_K) return -1;
    if (!x || !w || !du || !dx || !dw || !db) return -1;
    int nt = set_threads(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t d = 0; d < D; d++) {
        double sw[ORACLE_MAX_K];
        double sb = 0.0;
        for (int64_t k = 0; k < K; k++) sw[k] = 0.0;
        for (int64_t b = 0; b < B; b++) {
            for (int64_t t = 0; t < L; t++) dx[(b * L + t) * D + d] = 0.0;
            for (int64_t t = 0; t < L; t++) {
                const int64_t r = b * L + t;
                const double dc = (double)du[r * D + d] *
                                  silu_grad(conv_at(x, w, bias, L, D, K, b, t, d));
                sb += dc;
                for (int64_t k = 0; k < K && k <= t; k++) {
                    sw[k] += dc * (double)x[(r - k) * D + d];
                    dx[(r - k) * D + d] += dc * (double)w[d * K + k];
                }
            }
        }
        for (int64_t k = 0; k < K; k++) dw[d * K + k] = sw[k];
        db[d] = sb;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Mamba-2 state-space-dual scan (the recurrence that the pages' Mamba2Block
 * dispatches as ssd_chunk_forward, same package, src/model/mamba2_block.ts;
 * the pages show its buffers but not its arithmetic).  Plainest reading,
 * consistent with the Mamba-1 path of the same pages:
 *   H heads of P channels (x column h*P + p), G groups of N states sharing
 *   B and C (head h uses group h / (H / G), column g*N + n);
 *   dv = softplus(dt[r, h] + dt_bias[h]),  A_h = -exp(clamp(A_log[h], -10, 5))
 *   S_h[p, n] <- exp(dv A_h) S_h[p, n] + f x[r, h*P + p] B[r, g*N + n]
 *   with the input factor f = dv (EULER) or expm1(dv A_h) / A_h (ZOH), the
 *   two discretisations of the Mamba-1 path
 *   y[r, h*P + p] = sum_n C[r, g*N + n] S_h[p, n] + D[h] x[r, h*P + p]
 * State (B, H, P, N), starting at h0 or 0.  One (b, h) at a time, time in
 * order, fp64.                                                              */
int oracle_ssd_scan(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int disc,
                    const float* x, const float* dt, const float* A_log, const float* Bm,
                    const float* Cm, const float* Dv, const float* dt_bias, const float* h0,
                    double* y, double* h_last, int nthreads) {
    if (B < 0 || L < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return -1;
    if (disc != ORACLE_DISC_ZOH && disc != ORACLE_DISC_EULER) return -1;
    if (!x || !dt || !A_log || !Bm || !Cm || !y) return -1;
    const int64_t HP = H * P, GN = G * N, hpg = H / G;
    int nt = set_threads(nthreads);
    int err = 0;
#pragma omp parallel num_threads(nt)
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)(P * N));
        if (!S) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; bh++) {
            if (!S) continue;
            const int64_t b = bh / H, h = bh % H, g = h / hpg;
            const double A = a_cont((double)A_log[h]);
            const double bias = dt_bias ? (double)dt_bias[h] : 0.0;
            const double Dh = Dv ? (double)Dv[h] : 0.0;
            for (int64_t i = 0; i < P * N; i++)
                S[i] = h0 ? (double)h0[bh * P * N + i] : 0.0;
            for (int64_t t = 0; t < L; t++) {
                const int64_t r = b * L + t;
                const double dv = softplus((double)dt[r * H + h] + bias);
                const double a = exp(dv * A);
                const double f = b_bar(disc, dv, A, 1.0);
                for (int64_t p = 0; p < P; p++) {
                    const double xv = (double)x[r * HP + h * P + p];
                    double acc = Dh * xv;
                    for (int64_t n = 0; n < N; n++) {
                        double* s = &S[p * N + n];
                        *s = a * *s + f * xv * (double)Bm[r * GN + g * N + n];
                        acc += (double)Cm[r * GN + g * N + n] * *s;
                    }
                    y[r * HP + h * P + p] = acc;
                }
            }
            if (h_last)
                for (int64_t i = 0; i < P * N; i++) h_last[bh * P * N + i] = S[i];
        }
        free(S);
    }
    return err;
}

int oracle_abi_version(void) { return 1; }
