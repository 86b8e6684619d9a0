// step_kernel.hip -- one single-token recurrent step (decode) of the Mamba-1
// block core with carried state: the per-step update of mamba1CpuForward
// steps 4, 5, 8 and 9 (builderforce-memory-engine 2026.7.12 -> 2026.9.27,
// src/training/mamba1_cpu.ts) applied to one new input per sequence, with the
// conv window (the K-1 previous inputs, oldest first) and h carried in
// caller-owned buffers that are updated in place.
//
// HBM-bound: per (b, d) it reads and writes h (2 * 4N bytes) and the conv
// window (2 * 4(K-1) bytes) plus x, z, delta, y.  Lane = channel d: the N
// states of a lane are contiguous, so a wave moves 64 * 4N contiguous bytes
// with 16-byte vector accesses; B and C rows of a batch entry are
// wave-uniform scalar loads.
#include "device_math.h"
#include "launch.h"

namespace mss {
namespace {

constexpr float kSmallX = 0.015625f;          // same ZOH expm1 switch as the scan

template <int DISC, int KS, int NS>
__global__ __launch_bounds__(kWave) void step_kernel(StepArgs a) {
    constexpr int NR = NS > 0 ? NS : kMaxN;
    constexpr int KR = KS > 0 ? KS : kMaxK;
    const int N = NS > 0 ? NS : a.N;
    const int K = KS > 0 ? KS : a.K;
    const int64_t tiles = (a.D + kWave - 1) / kWave;
    const int64_t nblk = a.B * tiles;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t b = blk / tiles;
        const int64_t d_raw = (blk - b * tiles) * kWave + threadIdx.x;
        const bool valid = d_raw < a.D;
        const int64_t d = valid ? d_raw : a.D - 1;
        const int64_t bd = b * a.D + d;

        // conv over (window, x).  Registers hold the window newest first:
        // prev[k-1] = input k steps back = conv_state[K-1-k] (oldest-first
        // buffer), so every register index is a compile-time constant.
        const float xv = a.x[bd];
        float prev[KR > 1 ? KR - 1 : 1];
#pragma unroll
        for (int k = 1; k < KR; k++)
            prev[k - 1] = k < K ? a.conv_state[(b * (K - 1) + (K - 1 - k)) * a.D + d] : 0.0f;
        float acc = a.b_conv ? a.b_conv[d] : 0.0f;
        acc = __builtin_fmaf(a.w_conv[d * K], xv, acc);
#pragma unroll
        for (int k = 1; k < KR; k++)
            if (k < K) acc = __builtin_fmaf(a.w_conv[d * K + k], prev[k - 1], acc);
        const float u = silu(acc);
        const float dv = softplus(a.delta[bd]);

        float h[NR], A2[NR], Ai[NR];
        float* __restrict__ hp = a.h + bd * N;
        if constexpr (NS > 0 && NS % 4 == 0) {
#pragma unroll
            for (int n = 0; n < NR; n += 4) {
                const float4 v = *reinterpret_cast<const float4*>(hp + n);
                h[n] = v.x; h[n + 1] = v.y; h[n + 2] = v.z; h[n + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int n = 0; n < NR; n++) h[n] = n < N ? hp[n] : 0.0f;
        }
#pragma unroll
        for (int n = 0; n < NR; n++) {
            const float A = (NS > 0 || n < N) ? a_cont(a.A_log[d * N + n]) : -1.0f;
            A2[n] = A * kLog2e;
            Ai[n] = 1.0f / A;
        }
        const cfloat* Br = as_const(a.B_in + b * N);
        const cfloat* Cr = as_const(a.C_in + b * N);
        float yv = (a.D_vec ? a.D_vec[d] : 0.0f) * u;
        // The decay is applied as h + m h with m = expm1(dv A) (a cubic when
        // |dv A| < 2^-6): a nearly-integrating state keeps its accuracy over
        // any number of steps.  Memory-bound, so no fast path is needed.
        const float dvu = dv * u;
#pragma unroll
        for (int n = 0; n < NR; n++) {
            if (NS > 0 || n < N) {
                const float x2 = dv * A2[n];
                const float ab = ex2(x2);
                const float x = x2 * kLn2;
                const float p = x * __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 6.0f, 0.5f), 1.0f);
                const float m = __builtin_fabsf(x) < kSmallX ? p : ab - 1.0f;
                if constexpr (DISC == MSS_DISC_EULER) {
                    h[n] = __builtin_fmaf(dvu, Br[n], __builtin_fmaf(m, h[n], h[n]));
                } else {
                    const float kk = (u * Ai[n]) * Br[n];
                    h[n] = __builtin_fmaf(m, h[n] + kk, h[n]);
                }
                yv = __builtin_fmaf(Cr[n], h[n], yv);
            }
        }
        if (valid) {
            a.y[bd] = a.z ? yv * silu(a.z[bd]) : yv;
            if constexpr (NS > 0 && NS % 4 == 0) {
#pragma unroll
                for (int n = 0; n < NR; n += 4)
                    *reinterpret_cast<float4*>(hp + n) = make_float4(h[n], h[n + 1], h[n + 2], h[n + 3]);
            } else {
#pragma unroll
                for (int n = 0; n < NR; n++)
                    if (n < N) hp[n] = h[n];
            }
            // shifted window: position K-1-k now holds the input k-1 steps back
#pragma unroll
            for (int k = 1; k < KR; k++)
                if (k < K)
                    a.conv_state[(b * (K - 1) + (K - 1 - k)) * a.D + d] = k == 1 ? xv : prev[k >= 2 ? k - 2 : 0];
        }
    }
}

template <int DISC, int KS>
hipError_t launch_n(const StepArgs& a, unsigned grid, hipStream_t st) {
    if (a.N == 16)
        hipLaunchKernelGGL((step_kernel<DISC, KS, 16>), dim3(grid), dim3(kWave), 0, st, a);
    else
        hipLaunchKernelGGL((step_kernel<DISC, KS, 0>), dim3(grid), dim3(kWave), 0, st, a);
    return hipGetLastError();
}

template <int DISC>
hipError_t launch_k(const StepArgs& a, unsigned grid, hipStream_t st) {
    return a.K == 4 ? launch_n<DISC, 4>(a, grid, st) : launch_n<DISC, 0>(a, grid, st);
}

}  // namespace

hipError_t launch_step(const StepArgs& a, hipStream_t st) {
    const int64_t nblk = a.B * ((a.D + kWave - 1) / kWave);
    const unsigned grid = static_cast<unsigned>(nblk < (1 << 30) ? nblk : (1 << 30));
    return a.disc == MSS_DISC_EULER ? launch_k<MSS_DISC_EULER>(a, grid, st)
                                    : launch_k<MSS_DISC_ZOH>(a, grid, st);
}

}  // namespace mss
