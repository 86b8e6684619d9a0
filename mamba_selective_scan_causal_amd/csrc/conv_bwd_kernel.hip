// conv_bwd_kernel.hip -- backward of the causal depthwise conv1d + SiLU
// (mamba1CpuBackward, "SiLU" and "Depthwise causal conv1d" parts,
// builderforce-memory-engine 2026.7.12 -> 2026.9.27,
// src/training/mamba1_cpu.ts).  With c the conv output and
// dc = du * SiLU'(c):
//   dx[b,t,d] = sum_{k<K, t+k<L} dc[b,t+k,d] * wConv[d,k]
//   dwConv[d,k] = sum_{b,t>=k} dc[b,t,d] * x[b,t-k,d]
//   dbConv[d]   = sum_{b,t} dc[b,t,d]
//
// HBM-bound (x and du in, dx out: 12 bytes per element).  Lane = channel d;
// a wave walks 32-step runs with every load of a run issued before first
// use, recomputing c from x (and dc over the K-1 steps past the run that dx
// needs).  The dw / db sums stay in registers across all runs of the wave
// and are written once per wave; a second kernel adds the waves of a channel
// tile in a fixed order.  Each tap count 1..8 is its own instantiation, so
// no padded zero tap multiplies an input (0 * Inf would be NaN).
#include "device_math.h"
#include "launch_bwd.h"

namespace mss {
namespace {

constexpr int kRun = 32;
constexpr int kPartRows = kMaxK + 1;

__device__ __forceinline__ float silu_grad(float v) {
    const float s = rcp(1.0f + ex2(-kLog2e * v));
    return s * __builtin_fmaf(v, 1.0f - s, 1.0f);
}

// dx and the dw, db sums over the kRun steps of one run.  In the last run of
// a row (TAIL) the steps past the end take no part: the x repeated there may
// be non-finite, so they are skipped rather than multiplied by zero.  The
// guard is uniform across the wave; it is a separate instantiation so that
// full runs carry no per-step test.
// x at t0 - (KR - 1) .. t0 + kRun + KR - 2 and dc = du * SiLU'(c) at
// t0 .. t0 + kRun + KR - 2 for one run.  EDGE: the run touches an end of the
// row, so indices are clamped into it, x before the start is 0 and dc past
// the end is 0 (a select, not a product: the x repeated there may be
// non-finite).
template <int KR, bool EDGE>
__device__ __forceinline__ void load_run(const ConvBwdArgs& a, const float (&w)[KR], float bias,
                                         float (&xv)[kRun + 2 * (KR - 1)],
                                         float (&dc)[kRun + KR - 1], int64_t base, int64_t t0) {
    constexpr int NX = kRun + 2 * (KR - 1), NC = kRun + KR - 1;
    const int64_t L = a.L, D = a.D;
    float gv[NC];
    if (EDGE) {
#pragma unroll
        for (int i = 0; i < NX; i++) {
            const int64_t t = t0 - (KR - 1) + i;
            const int64_t tc = t < 0 ? 0 : (t < L ? t : L - 1);
            const float v = a.x[base + tc * D];
            xv[i] = t >= 0 ? v : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < NC; i++) {
            const int64_t t = t0 + i;
            const float v = a.du[base + (t < L ? t : L - 1) * D];
            gv[i] = t < L ? v : 0.0f;
        }
    } else {
        const float* xp = a.x + base + (t0 - (KR - 1)) * D;
        const float* gp = a.du + base + t0 * D;
#pragma unroll
        for (int i = 0; i < NX; i++) xv[i] = xp[i * D];
#pragma unroll
        for (int i = 0; i < NC; i++) gv[i] = gp[i * D];
    }
#pragma unroll
    for (int i = 0; i < NC; i++) {
        float c = bias;
#pragma unroll
        for (int k = 0; k < KR; k++) c = __builtin_fmaf(w[k], xv[i + KR - 1 - k], c);
        const float v = gv[i] * silu_grad(c);
        dc[i] = EDGE && t0 + i >= L ? 0.0f : v;
    }
}

template <int KR, bool TAIL>
__device__ __forceinline__ void run_steps(const ConvBwdArgs& a, const float (&w)[KR],
                                          const float (&xv)[kRun + 2 * (KR - 1)],
                                          const float (&dc)[kRun + KR - 1], float (&sw)[KR],
                                          float& sb, int64_t base, int64_t t0, bool live) {
#pragma unroll
    for (int i = 0; i < kRun; i++) {
        const int64_t t = t0 + i;
        if (TAIL && t >= a.L) continue;
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < KR; k++) acc = __builtin_fmaf(w[k], dc[i + k], acc);
        // dx is written once and not read here again: the nontemporal
        // (streaming) hint measured 0.491 -> 0.475 ms on B4 L8192 D5120
        // (the same hint on the x and du loads, which neighbouring runs
        // re-read, 0.486 ms), bit-identical
        if (live) __builtin_nontemporal_store(acc, &a.dx[base + t * a.D]);
        sb += dc[i];
#pragma unroll
        for (int k = 0; k < KR; k++) sw[k] = __builtin_fmaf(dc[i], xv[i + KR - 1 - k], sw[k]);
    }
}

template <int K>
__global__ __launch_bounds__(kWave) void conv_bwd_kernel(ConvBwdArgs a) {
    constexpr int KR = K;
    const int64_t L = a.L, D = a.D;
    const int64_t runs = (L + kRun - 1) / kRun;
    const int64_t tile = blockIdx.x / a.groups;
    const int64_t g = blockIdx.x - tile * a.groups;
    const int64_t d_raw = tile * kWave + threadIdx.x;
    const bool live = d_raw < D;
    const int64_t d = live ? d_raw : D - 1;

    float w[KR];
#pragma unroll
    for (int k = 0; k < KR; k++) w[k] = a.w_conv[d * K + k];
    const float bias = a.b_conv ? a.b_conv[d] : 0.0f;
    float sw[KR], sb = 0.0f;
#pragma unroll
    for (int k = 0; k < KR; k++) sw[k] = 0.0f;

    constexpr int NX = kRun + 2 * (KR - 1);   // x at t0-(KR-1) .. t0+kRun+KR-2
    constexpr int NC = kRun + KR - 1;         // dc at t0 .. t0+kRun+KR-2
    for (int64_t job = g; job < a.B * runs; job += a.groups) {
        const int64_t b = job / runs;
        const int64_t t0 = (job - b * runs) * kRun;
        const int64_t base = b * L * D + d;
        float xv[NX], dc[NC];
        // runs that touch neither end of the row load without clamps
        if (t0 >= KR - 1 && t0 + NC <= L)
            load_run<KR, false>(a, w, bias, xv, dc, base, t0);
        else
            load_run<KR, true>(a, w, bias, xv, dc, base, t0);
        if (t0 + kRun <= L)
            run_steps<KR, false>(a, w, xv, dc, sw, sb, base, t0, live);
        else
            run_steps<KR, true>(a, w, xv, dc, sw, sb, base, t0, live);
    }
    float* p = a.part + blockIdx.x * static_cast<int64_t>(kPartRows * kWave) + threadIdx.x;
#pragma unroll
    for (int k = 0; k < KR; k++) p[k * kWave] = sw[k];
    p[K * kWave] = sb;
}

// One thread per (channel, row): row k < K is dw[d, k], row K is db[d]; the
// groups of the channel's tile are added in order.
__global__ __launch_bounds__(256) void conv_bwd_reduce_kernel(ConvBwdArgs a) {
    const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    const int64_t rows = a.K + 1;
    if (i >= a.D * rows) return;
    const int64_t d = i / rows;
    const int k = static_cast<int>(i - d * rows);
    if (k == a.K && !a.db) return;
    const int64_t tile = d / kWave, lane = d - tile * kWave;
    const float* p = a.part + (tile * a.groups * kPartRows + k) * kWave + lane;
    float acc = 0.0f;
    for (int64_t g = 0; g < a.groups; g++) acc += p[g * kPartRows * kWave];
    if (k < a.K)
        a.dw[d * a.K + k] = acc;
    else
        a.db[d] = acc;
}

}  // namespace

hipError_t launch_conv1d_silu_bwd(const ConvBwdArgs& a, hipStream_t st) {
    const int64_t tiles = (a.D + kWave - 1) / kWave;
    const unsigned grid = static_cast<unsigned>(tiles * a.groups);
    switch (a.K) {
#define MSS_CONV_BWD_CASE(k)                                                        \
    case k:                                                                         \
        hipLaunchKernelGGL(conv_bwd_kernel<k>, dim3(grid), dim3(kWave), 0, st, a); \
        break;
        MSS_CONV_BWD_CASE(1) MSS_CONV_BWD_CASE(2) MSS_CONV_BWD_CASE(3) MSS_CONV_BWD_CASE(4)
        MSS_CONV_BWD_CASE(5) MSS_CONV_BWD_CASE(6) MSS_CONV_BWD_CASE(7) MSS_CONV_BWD_CASE(8)
#undef MSS_CONV_BWD_CASE
        default:
            return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(conv_bwd_reduce_kernel,
                       dim3(static_cast<unsigned>((a.D * (a.K + 1) + 255) / 256)), dim3(256), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace mss
