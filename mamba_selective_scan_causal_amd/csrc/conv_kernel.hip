// conv_kernel.hip -- causal depthwise conv1d + SiLU (mamba1CpuForward steps 4
// and 5, builderforce-memory-engine 2026.7.12 -> 2026.9.27,
// src/training/mamba1_cpu.ts; GPU dispatch conv1d_forward in
// src/model/mamba1_block.ts of 2026.7.14 -> 2026.9.28):
//   u[b,t,d] = SiLU(bConv[d] + sum_{k<K, k<=t} wConv[d*K+k] * x[b,t-k,d])
//
// HBM-bound (8 bytes per element).  Lane = channel d, so each time row is one
// coalesced 256-byte segment per wave; each lane walks kRun consecutive steps
// with the K-1 previous inputs in registers, and issues all of its loads
// (the K-1 halo rows plus its kRun rows) before the first use.  Each tap
// count 1..8 is its own instantiation, so only the K real taps are summed
// (a padded zero tap would still multiply an older input, and 0 * Inf is
// NaN where the K-tap sum is finite).
#include "device_math.h"
#include "launch.h"

namespace mss {
namespace {

constexpr int kRun = 32;

template <int K>
__global__ __launch_bounds__(kWave) void conv_kernel(const float* __restrict__ x,
                                                     const float* __restrict__ w_conv,
                                                     const float* __restrict__ b_conv,
                                                     float* __restrict__ u, int64_t B, int64_t L,
                                                     int64_t D) {
    constexpr int KR = K;
    const int64_t tiles = (D + kWave - 1) / kWave;
    const int64_t runs = (L + kRun - 1) / kRun;
    const int64_t nblk = B * runs * tiles;
    // Block id = (b * runs + run) * tiles + tile: neighbouring waves read
    // neighbouring 256-byte pieces of the same rows.
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t tile = blk % tiles;
        const int64_t run = (blk / tiles) % runs;
        const int64_t b = blk / (tiles * runs);
        const int64_t d_raw = tile * kWave + threadIdx.x;
        const bool valid = d_raw < D;
        const int64_t d = valid ? d_raw : D - 1;
        const int64_t t0 = run * kRun;
        const int64_t base = b * L * D + d;

        float w[KR];
#pragma unroll
        for (int k = 0; k < KR; k++) w[k] = w_conv[d * K + k];
        const float bias = b_conv ? b_conv[d] : 0.0f;

        // v[i] = x at t0 - (KR-1) + i; zero before the start of the batch row.
        float v[kRun + KR - 1];
#pragma unroll
        for (int i = 0; i < kRun + KR - 1; i++) {
            const int64_t t = t0 - (KR - 1) + i;
            const int64_t tc = t < 0 ? 0 : (t < L ? t : L - 1);
            const float xv = x[base + tc * D];
            v[i] = t >= 0 ? xv : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kRun; i++) {
            const int64_t t = t0 + i;
            float acc = bias;
#pragma unroll
            for (int k = 0; k < KR; k++) acc = __builtin_fmaf(w[k], v[i + KR - 1 - k], acc);
            // u is not read again here: stored with the nontemporal
            // (streaming) hint, 258.5 -> 250.4 us on B4 L8192 D5120
            if (valid && t < L) __builtin_nontemporal_store(silu(acc), &u[base + t * D]);
        }
    }
}

__global__ __launch_bounds__(256) void state_init_kernel(const float* __restrict__ h0,
                                                         float* __restrict__ out, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        out[i] = h0 ? h0[i] : 0.0f;
}

}  // namespace

hipError_t launch_conv1d_silu(const ConvArgs& a, hipStream_t st) {
    const int64_t nblk = a.B * ((a.L + kRun - 1) / kRun) * ((a.D + kWave - 1) / kWave);
    const unsigned grid = static_cast<unsigned>(nblk < (1 << 30) ? nblk : (1 << 30));
    switch (a.K) {
#define MSS_CONV_CASE(k)                                                                     \
    case k:                                                                                  \
        hipLaunchKernelGGL(conv_kernel<k>, dim3(grid), dim3(kWave), 0, st, a.x, a.w_conv,   \
                           a.b_conv, a.u, a.B, a.L, a.D);                                    \
        break;
        MSS_CONV_CASE(1) MSS_CONV_CASE(2) MSS_CONV_CASE(3) MSS_CONV_CASE(4)
        MSS_CONV_CASE(5) MSS_CONV_CASE(6) MSS_CONV_CASE(7) MSS_CONV_CASE(8)
#undef MSS_CONV_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_state_init(const float* h0, float* h_last, int64_t count, hipStream_t st) {
    const int64_t nblk = (count + 255) / 256;
    const unsigned grid = static_cast<unsigned>(nblk < (1 << 30) ? nblk : (1 << 30));
    hipLaunchKernelGGL(state_init_kernel, dim3(grid), dim3(256), 0, st, h0, h_last, count);
    return hipGetLastError();
}

}  // namespace mss
