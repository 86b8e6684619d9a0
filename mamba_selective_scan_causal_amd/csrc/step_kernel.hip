// step_kernel.hip -- one single-token recurrent step (decode) of the Mamba-1
// block core with carried state: the per-step update of mamba1CpuForward
// steps 4, 5, 8 and 9 (builderforce-memory-engine 2026.7.12 -> 2026.9.27,
// src/training/mamba1_cpu.ts) applied to one new input per sequence, with the
// conv window (the K-1 previous inputs, oldest first) and h carried in
// caller-owned buffers that are updated in place.
//
// HBM-bound: per (b, d) it reads and writes h (2 * 4N bytes) and the conv
// window (2 * 4(K-1) bytes) plus x, z, delta, y.  A lane owns one channel and
// its N states, so a wave's h block (64 channels) is 64 * 4N contiguous
// bytes.  With N = 16 that block moves in 16-byte pieces with consecutive
// lanes on consecutive pieces (each access one contiguous 1 KB): piece i of
// lane (m, s) = (lane / 4, lane % 4) holds states 4 s .. 4 s + 3 of channel
// 16 i + m, so lane (m, s) is given channel 16 s + m, and a 4 x 4 transpose
// of the pieces inside each quad of lanes (DPP) puts a channel's 16 states
// in its lane.  B and C rows of a batch entry are wave-uniform.
#include "device_math.h"
#include "launch.h"

namespace mss {
namespace {

constexpr float kSmallX = 0.015625f;          // same ZOH expm1 switch as the scan

// Batch rows per wave: the per-channel parameters (A, 1/A, conv taps) are
// loaded and transformed once for kRows rows, and all loads of the rows are
// issued before any arithmetic so that their latencies overlap.
constexpr int kRows = 2;

// The value of lane ^ B (B = 1 or 2) inside its quad (DPP quad_perm).
template <int B>
__device__ __forceinline__ float quad_xor(float v) {
    constexpr int ctrl = B == 1 ? 0xb1 : 0x4e;   // [1,0,3,2] or [2,3,0,1]
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xf, 0xf, true));
}

// One level of the in-quad transpose of v[piece][component]: the lanes whose
// bit B is clear keep pieces without bit B and trade the others with lane ^ B.
template <int B>
__device__ __forceinline__ void quad_trade(float (&v)[4][4]) {
    const bool hi = (threadIdx.x & B) != 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (i & B) continue;
        const int j = i | B;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float recv = quad_xor<B>(hi ? v[i][k] : v[j][k]);
            if (hi)
                v[i][k] = recv;
            else
                v[j][k] = recv;
        }
    }
}

// Lane g of a quad ends with piece i = lane i's piece g (its own inverse).
__device__ __forceinline__ void quad_transpose(float (&v)[4][4]) {
    quad_trade<1>(v);
    quad_trade<2>(v);
}

template <int DISC, int KS, int NS>
__global__ __launch_bounds__(kWave) void step_kernel(StepArgs a) {
    constexpr int NR = NS > 0 ? NS : kMaxN;
    constexpr int KR = KS > 0 ? KS : kMaxK;
    constexpr bool kStageBC = NS == 16 && kRows * 32 == kWave;
    __shared__ __align__(16) float bcs[kWave];
    const int N = NS > 0 ? NS : a.N;
    const int K = KS > 0 ? KS : a.K;
    const int64_t tiles = (a.D + kWave - 1) / kWave;
    const int64_t groups = (a.B + kRows - 1) / kRows;
    const int64_t nblk = groups * tiles;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t g = blk / tiles;
        const int64_t d0 = (blk - g * tiles) * kWave;   // first channel of the tile
        // N = 16: lane (m, s) owns channel 16 s + m (see the file header)
        const int64_t d_raw =
            d0 + (kStageBC ? 16 * (threadIdx.x & 3u) + (threadIdx.x >> 2) : threadIdx.x);
        const bool valid = d_raw < a.D;
        const int64_t d = valid ? d_raw : a.D - 1;
        int64_t bs[kRows];
        bool live[kRows];
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            const int64_t b = g * kRows + r;
            live[r] = b < a.B;            // wave-uniform
            bs[r] = live[r] ? b : a.B - 1;
        }

        // --- every load first: B/C rows, per-row inputs and state, then the
        // per-channel parameters.  With N = 16 the B and C rows of the
        // wave's kRows batch entries are exactly one float per lane: loaded
        // as one vector load together with the rest, staged through LDS and
        // read back as broadcasts.
        float bc = 0.0f;
        if constexpr (kStageBC) {
            const uint32_t l = threadIdx.x, r = l / 32, j = l % 32;
            bc = j < 16 ? a.B_in[bs[r] * 16 + j] : a.C_in[bs[r] * 16 + (j - 16)];
        }
        float xv[kRows], dl[kRows], zv[kRows], h[kRows][NR];
        float prev[kRows][KR > 1 ? KR - 1 : 1];   // prev[r][k-1]: input k steps back
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            const int64_t bd = bs[r] * a.D + d;
            xv[r] = a.x[bd];
            dl[r] = a.delta[bd];
            zv[r] = a.z ? a.z[bd] : 0.0f;
#pragma unroll
            for (int k = 1; k < KR; k++)
                prev[r][k - 1] =
                    k < K ? a.conv_state[(bs[r] * (K - 1) + (K - 1 - k)) * a.D + d] : 0.0f;
            if constexpr (kStageBC) {
                // piece q = 64 i + lane of the row's block: channel d0 + q / 4
                const float4* src =
                    reinterpret_cast<const float4*>(a.h + (bs[r] * a.D + d0) * 16);
                float v[4][4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int q = i * kWave + static_cast<int>(threadIdx.x);
                    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (d0 + q / 4 < a.D) t = src[q];
                    v[i][0] = t.x; v[i][1] = t.y; v[i][2] = t.z; v[i][3] = t.w;
                }
                quad_transpose(v);
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int k = 0; k < 4; k++) h[r][4 * i + k] = v[i][k];
            } else if constexpr (NS > 0 && NS % 4 == 0) {
                const float* hp = a.h + bd * N;
#pragma unroll
                for (int n = 0; n < NR; n += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(hp + n);
                    h[r][n] = v.x; h[r][n + 1] = v.y; h[r][n + 2] = v.z; h[r][n + 3] = v.w;
                }
            } else {
                const float* hp = a.h + bd * N;
#pragma unroll
                for (int n = 0; n < NR; n++) h[r][n] = n < N ? hp[n] : 0.0f;
            }
        }
        float A2[NR], Ai[NR], w[KR];
#pragma unroll
        for (int n = 0; n < NR; n++) {
            const float A = (NS > 0 || n < N) ? a_cont_fast(a.A_log[d * N + n]) : -1.0f;
            A2[n] = A * kLog2e;
            Ai[n] = rcp(A);
        }
#pragma unroll
        for (int k = 0; k < KR; k++) w[k] = k < K ? a.w_conv[d * K + k] : 0.0f;
        const float bias = a.b_conv ? a.b_conv[d] : 0.0f;
        const float dvec = a.D_vec ? a.D_vec[d] : 0.0f;

        float Bv[kRows][NR], Cv[kRows][NR];
        if constexpr (kStageBC) {
            bcs[threadIdx.x] = bc;       // one wave per workgroup: program order suffices
            const float4* q = reinterpret_cast<const float4*>(bcs);
#pragma unroll
            for (int r = 0; r < kRows; r++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float4 bq = q[r * 8 + i], cq = q[r * 8 + 4 + i];
                    Bv[r][4 * i] = bq.x; Bv[r][4 * i + 1] = bq.y;
                    Bv[r][4 * i + 2] = bq.z; Bv[r][4 * i + 3] = bq.w;
                    Cv[r][4 * i] = cq.x; Cv[r][4 * i + 1] = cq.y;
                    Cv[r][4 * i + 2] = cq.z; Cv[r][4 * i + 3] = cq.w;
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < kRows; r++) {
                const cfloat* Br = as_const(a.B_in + bs[r] * N);
                const cfloat* Cr = as_const(a.C_in + bs[r] * N);
#pragma unroll
                for (int n = 0; n < NR; n++) {
                    Bv[r][n] = n < N ? Br[n] : 0.0f;
                    Cv[r][n] = n < N ? Cr[n] : 0.0f;
                }
            }
        }

#pragma unroll
        for (int r = 0; r < kRows; r++) {
            if (!live[r]) continue;
            // conv over (window, x): tap 0 is the new input
            float acc = __builtin_fmaf(w[0], xv[r], bias);
#pragma unroll
            for (int k = 1; k < KR; k++)
                if (k < K) acc = __builtin_fmaf(w[k], prev[r][k - 1], acc);
            const float u = silu(acc);
            const float dv = softplus(dl[r]);
            float yv = dvec * u;
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
                    const float p =
                        x * __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 6.0f, 0.5f), 1.0f);
                    const float m = __builtin_fabsf(x) < kSmallX ? p : ab - 1.0f;
                    if constexpr (DISC == MSS_DISC_EULER) {
                        h[r][n] = __builtin_fmaf(dvu, Bv[r][n], __builtin_fmaf(m, h[r][n], h[r][n]));
                    } else {
                        const float kk = (u * Ai[n]) * Bv[r][n];
                        h[r][n] = __builtin_fmaf(m, h[r][n] + kk, h[r][n]);
                    }
                    yv = __builtin_fmaf(Cv[r][n], h[r][n], yv);
                }
            }
            if constexpr (kStageBC) {
                // back to pieces (every lane of the quad takes part), then
                // one contiguous 1 KB store per piece index
                float v[4][4];
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int k = 0; k < 4; k++) v[i][k] = h[r][4 * i + k];
                quad_transpose(v);
                float4* dst = reinterpret_cast<float4*>(a.h + (bs[r] * a.D + d0) * 16);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int q = i * kWave + static_cast<int>(threadIdx.x);
                    if (d0 + q / 4 < a.D) dst[q] = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
                }
            }
            if (valid) {
                const int64_t bd = bs[r] * a.D + d;
                a.y[bd] = a.z ? yv * silu(zv[r]) : yv;
                float* hp = a.h + bd * N;
                if constexpr (kStageBC) {
                    // stored above
                } else if constexpr (NS > 0 && NS % 4 == 0) {
#pragma unroll
                    for (int n = 0; n < NR; n += 4)
                        *reinterpret_cast<float4*>(hp + n) =
                            make_float4(h[r][n], h[r][n + 1], h[r][n + 2], h[r][n + 3]);
                } else {
#pragma unroll
                    for (int n = 0; n < NR; n++)
                        if (n < N) hp[n] = h[r][n];
                }
                // shifted window: position K-1-k now holds the input k-1 steps back
#pragma unroll
                for (int k = 1; k < KR; k++)
                    if (k < K)
                        a.conv_state[(bs[r] * (K - 1) + (K - 1 - k)) * a.D + d] =
                            k == 1 ? xv[r] : prev[r][k >= 2 ? k - 2 : 0];
            }
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
    const int64_t nblk = ((a.B + kRows - 1) / kRows) * ((a.D + kWave - 1) / kWave);
    const unsigned grid = static_cast<unsigned>(nblk < (1 << 30) ? nblk : (1 << 30));
    return a.disc == MSS_DISC_EULER ? launch_k<MSS_DISC_EULER>(a, grid, st)
                                    : launch_k<MSS_DISC_ZOH>(a, grid, st);
}

}  // namespace mss
