// step_kernel.hip -- one single-token recurrent step (decode) of the Mamba-1
// block core with carried state: the per-step update of mamba1CpuForward
// steps 4, 5, 8 and 9 (builderforce-memory-engine 2026.7.12 -> 2026.9.27,
// src/training/mamba1_cpu.ts) applied to one new input per sequence, with the
// conv window (the K-1 previous inputs, oldest first) and h carried in
// caller-owned buffers that are updated in place.
//
// HBM-bound: per (b, d) it reads and writes h (2 * 4N bytes) and the conv
// window (2 * 4(K-1) bytes) plus x, z, delta, y.
//
// N = 16 (step16_kernel): a wave keeps one tile of 64 channels -- their A,
// 1/A and conv taps are computed once -- and takes batch rows two at a time
// from a set of groups shared evenly between the waves of that tile.  h,
// like A_log, is moved in 16-byte pieces with consecutive lanes on
// consecutive pieces, so every h access is one contiguous 1 KB.  Lane
// (m, s) = (lane / 4, lane % 4) holds piece i = 0..3 of the block: states
// 4 s .. 4 s + 3 of channel 16 i + m, and updates those 16 (channel, state)
// pairs in place.  The per-channel scalars are computed once, by the lane
// that owns the channel (lane (m, s) owns channel 16 s + m), and handed to
// the quad by DPP broadcasts; the quad's partial sums of C h are reduced
// back to the owner by a two-level exchange.  Other N (step_kernel): one
// channel and its N states per lane.
#include "device_math.h"
#include "launch.h"

namespace mss {
namespace {

constexpr float kSmallX = 0.015625f;          // same ZOH expm1 switch as the scan

// Batch rows per group: all loads of a group's rows are issued before any
// arithmetic so that their latencies overlap.
constexpr int kRows = 2;

// Accesses with the nontemporal (streaming) cache hint.  In step16_kernel,
// x, z, delta, y and the state h go through these; the conv window does not.
// Measured on B256 D5120 (64 consecutive steps, in place): 36.9 us per step
// against 42.7 us with every access cached, 45.8 against 52.9 us from a cold
// last-level cache; h alone hinted ran 38.3 us, the activations alone
// 42.5 us, and everything including the window 39.9 us.  Results are
// bit-identical: the hint changes caching only.
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float ld_nt(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 ld_nt(const float4* p) {
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(float4* p, float4 v) {
    __builtin_nontemporal_store(f4v{v.x, v.y, v.z, v.w}, reinterpret_cast<f4v*>(p));
}

// The value of lane ^ B (B = 1 or 2) inside its quad (DPP quad_perm).
template <int B>
__device__ __forceinline__ float quad_xor(float v) {
    constexpr int ctrl = B == 1 ? 0xb1 : 0x4e;   // [1,0,3,2] or [2,3,0,1]
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xf, 0xf, true));
}

// The value of lane I of this lane's quad (DPP quad_perm [I,I,I,I]).
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
    constexpr int ctrl = I * 0x55;
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xf, 0xf, true));
}

// p[i] of the four lanes of a quad summed, lane s receiving the sum for
// i = s: two exchange levels that each keep half of the values (selected by
// lane bits 0, then 1) and add the partner's other half.
__device__ __forceinline__ float quad_reduce_scatter(const float (&p)[4]) {
    const bool b0 = (threadIdx.x & 1u) != 0, b1 = (threadIdx.x & 2u) != 0;
    float w[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const float keep = b0 ? p[2 * t + 1] : p[2 * t];
        const float send = b0 ? p[2 * t] : p[2 * t + 1];
        w[t] = keep + quad_xor<1>(send);
    }
    const float keep = b1 ? w[1] : w[0];
    const float send = b1 ? w[0] : w[1];
    return keep + quad_xor<2>(send);
}

// One step of one (channel, state) pair: the decay applied as h + m h with
// m = expm1(dv A) (a cubic when |dv A| < 2^-6), so a nearly-integrating state
// keeps its accuracy over any number of steps (memory-bound: no fast path).
template <int DISC>
__device__ __forceinline__ float step_state(float h, float dv, float A2, float Ai, float u,
                                            float dvu, float Bn) {
    const float x2 = dv * A2;
    const float ab = ex2(x2);
    const float x = x2 * kLn2;
    const float p = x * __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 6.0f, 0.5f), 1.0f);
    const float m = __builtin_fabsf(x) < kSmallX ? p : ab - 1.0f;
    if constexpr (DISC == MSS_DISC_EULER) {
        return __builtin_fmaf(dvu, Bn, __builtin_fmaf(m, h, h));
    } else {
        const float kk = (u * Ai) * Bn;
        return __builtin_fmaf(m, h + kk, h);
    }
}

// N = 16: see the file header for the lane layout.
template <int DISC, int KS>
__global__ __launch_bounds__(kWave) void step16_kernel(StepArgs a) {
    constexpr int KR = KS > 0 ? KS : kMaxK;
    const int K = KS > 0 ? KS : a.K;
    __shared__ __align__(16) float bcs[kRows * 32];   // per row: B (16), C (16)
    const uint32_t lane = threadIdx.x, m = lane >> 2, s = lane & 3u;
    const int64_t tiles = (a.D + kWave - 1) / kWave;
    const int64_t groups = (a.B + kRows - 1) / kRows;
    // wave w keeps channel tile w % tiles and takes the batch groups
    // w / tiles, + G, + 2 G, ... (the grid is tiles * G waves)
    const int64_t G = gridDim.x / tiles;
    const int64_t d0 = (blockIdx.x % tiles) * kWave;   // first channel of the tile
    const int64_t d_own = d0 + 16 * s + m;             // the channel this lane owns
    const bool valid = d_own < a.D;
    const int64_t d = valid ? d_own : a.D - 1;
    // piece i of this lane: channel d0 + 16 i + m, states 4 s .. 4 s + 3
    bool pvalid[4];
#pragma unroll
    for (int i = 0; i < 4; i++) pvalid[i] = d0 + 16 * i + m < a.D;
    // A of the lane's 16 (channel, state) pairs, laid out like h
    float A2[4][4], Ai[4][4];
    {
        const float4* src = reinterpret_cast<const float4*>(a.A_log + d0 * 16);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
            if (pvalid[i]) t = src[i * kWave + lane];
            const float al[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float A = pvalid[i] ? a_cont_fast(al[k]) : -1.0f;
                A2[i][k] = A * kLog2e;
                Ai[i][k] = rcp(A);
            }
        }
    }
    float w[KR];
#pragma unroll
    for (int k = 0; k < KR; k++) w[k] = k < K ? a.w_conv[d * K + k] : 0.0f;
    const float bias = a.b_conv ? a.b_conv[d] : 0.0f;
    const float dvec = a.D_vec ? a.D_vec[d] : 0.0f;
    for (int64_t g = blockIdx.x / tiles; g < groups; g += G) {
        int64_t bs[kRows];
        bool live[kRows];
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            const int64_t b = g * kRows + r;
            live[r] = b < a.B;            // wave-uniform
            bs[r] = live[r] ? b : a.B - 1;
        }

        // --- every load first.  B and C rows of the kRows batch entries are
        // one float per lane, staged through LDS.
        {
            const uint32_t r = lane / 32, j = lane % 32;
            bcs[lane] = j < 16 ? a.B_in[bs[r] * 16 + j] : a.C_in[bs[r] * 16 + (j - 16)];
        }
        float xv[kRows], dl[kRows], zv[kRows], h[kRows][4][4];
        float prev[kRows][KR > 1 ? KR - 1 : 1];   // prev[r][k-1]: input k steps back
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            const int64_t bd = bs[r] * a.D + d;
            xv[r] = ld_nt(a.x + bd);
            dl[r] = ld_nt(a.delta + bd);
            zv[r] = a.z ? ld_nt(a.z + bd) : 0.0f;
#pragma unroll
            for (int k = 1; k < KR; k++)
                prev[r][k - 1] =
                    k < K ? a.conv_state[(bs[r] * (K - 1) + (K - 1 - k)) * a.D + d] : 0.0f;
            const float4* src = reinterpret_cast<const float4*>(a.h + (bs[r] * a.D + d0) * 16);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
                if (pvalid[i]) t = ld_nt(src + i * kWave + lane);
                h[r][i][0] = t.x; h[r][i][1] = t.y; h[r][i][2] = t.z; h[r][i][3] = t.w;
            }
        }
        __syncthreads();
        float Bv[kRows][4], Cv[kRows][4];
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            const float4 bq = reinterpret_cast<const float4*>(bcs)[r * 8 + s];
            const float4 cq = reinterpret_cast<const float4*>(bcs)[r * 8 + 4 + s];
            Bv[r][0] = bq.x; Bv[r][1] = bq.y; Bv[r][2] = bq.z; Bv[r][3] = bq.w;
            Cv[r][0] = cq.x; Cv[r][1] = cq.y; Cv[r][2] = cq.z; Cv[r][3] = cq.w;
        }

#pragma unroll
        for (int r = 0; r < kRows; r++) {
            if (!live[r]) continue;
            // the owned channel's input: conv over (window, x), tap 0 the new one
            float acc = __builtin_fmaf(w[0], xv[r], bias);
#pragma unroll
            for (int k = 1; k < KR; k++)
                if (k < K) acc = __builtin_fmaf(w[k], prev[r][k - 1], acc);
            const float u = silu(acc);
            const float dv = softplus(dl[r]);
            // u and dv of the channels of pieces 0..3 (owned by quad lanes 0..3)
            const float ui[4] = {quad_bcast<0>(u), quad_bcast<1>(u), quad_bcast<2>(u),
                                 quad_bcast<3>(u)};
            const float di[4] = {quad_bcast<0>(dv), quad_bcast<1>(dv), quad_bcast<2>(dv),
                                 quad_bcast<3>(dv)};
            float py[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float dvu = di[i] * ui[i];
                float acc_y = 0.0f;
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    h[r][i][k] = step_state<DISC>(h[r][i][k], di[i], A2[i][k], Ai[i][k], ui[i],
                                                  dvu, Bv[r][k]);
                    acc_y = __builtin_fmaf(Cv[r][k], h[r][i][k], acc_y);
                }
                py[i] = acc_y;
            }
            const float yv = __builtin_fmaf(dvec, u, quad_reduce_scatter(py));
            float4* dst = reinterpret_cast<float4*>(a.h + (bs[r] * a.D + d0) * 16);
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (pvalid[i])
                    st_nt(dst + i * kWave + lane,
                          make_float4(h[r][i][0], h[r][i][1], h[r][i][2], h[r][i][3]));
            if (valid) {
                const int64_t bd = bs[r] * a.D + d;
                st_nt(a.y + bd, a.z ? yv * silu(zv[r]) : yv);
                // shifted window: position K-1-k now holds the input k-1 steps back
#pragma unroll
                for (int k = 1; k < KR; k++)
                    if (k < K)
                        a.conv_state[(bs[r] * (K - 1) + (K - 1 - k)) * a.D + d] =
                            k == 1 ? xv[r] : prev[r][k >= 2 ? k - 2 : 0];
            }
        }
        __syncthreads();   // the next group's B/C rows reuse bcs
    }
}

// Other N: one channel and its N states per lane.
template <int DISC, int KS>
__global__ __launch_bounds__(kWave) void step_kernel(StepArgs a) {
    constexpr int NR = kMaxN;
    constexpr int KR = KS > 0 ? KS : kMaxK;
    const int N = a.N;
    const int K = KS > 0 ? KS : a.K;
    const int64_t tiles = (a.D + kWave - 1) / kWave;
    const int64_t groups = (a.B + kRows - 1) / kRows;
    const int64_t nblk = groups * tiles;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t g = blk / tiles;
        const int64_t d_raw = (blk - g * tiles) * kWave + threadIdx.x;
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
        // every load first, then the per-channel parameters
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
            const float* hp = a.h + bd * N;
#pragma unroll
            for (int n = 0; n < NR; n++) h[r][n] = n < N ? hp[n] : 0.0f;
        }
        float A2[NR], Ai[NR], w[KR];
#pragma unroll
        for (int n = 0; n < NR; n++) {
            const float A = n < N ? a_cont_fast(a.A_log[d * N + n]) : -1.0f;
            A2[n] = A * kLog2e;
            Ai[n] = rcp(A);
        }
#pragma unroll
        for (int k = 0; k < KR; k++) w[k] = k < K ? a.w_conv[d * K + k] : 0.0f;
        const float bias = a.b_conv ? a.b_conv[d] : 0.0f;
        const float dvec = a.D_vec ? a.D_vec[d] : 0.0f;

#pragma unroll
        for (int r = 0; r < kRows; r++) {
            if (!live[r]) continue;
            const cfloat* Br = as_const(a.B_in + bs[r] * N);
            const cfloat* Cr = as_const(a.C_in + bs[r] * N);
            // conv over (window, x): tap 0 is the new input
            float acc = __builtin_fmaf(w[0], xv[r], bias);
#pragma unroll
            for (int k = 1; k < KR; k++)
                if (k < K) acc = __builtin_fmaf(w[k], prev[r][k - 1], acc);
            const float u = silu(acc);
            const float dv = softplus(dl[r]);
            const float dvu = dv * u;
            float yv = dvec * u;
#pragma unroll
            for (int n = 0; n < NR; n++) {
                if (n < N) {
                    h[r][n] = step_state<DISC>(h[r][n], dv, A2[n], Ai[n], u, dvu, Br[n]);
                    yv = __builtin_fmaf(Cr[n], h[r][n], yv);
                }
            }
            if (valid) {
                const int64_t bd = bs[r] * a.D + d;
                a.y[bd] = a.z ? yv * silu(zv[r]) : yv;
                float* hp = a.h + bd * N;
#pragma unroll
                for (int n = 0; n < NR; n++)
                    if (n < N) hp[n] = h[r][n];
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
    if (a.N == 16) {
        // tiles x G waves, G batch-group slots per tile: about 3072 waves (three
        // per SIMD), each taking the same number of groups
        const int64_t tiles = (a.D + kWave - 1) / kWave;
        const int64_t groups = (a.B + kRows - 1) / kRows;
        int64_t G = (3072 + tiles - 1) / tiles;
        if (G > groups) G = groups;
        if (G < 1) G = 1;
        const int64_t per = (groups + G - 1) / G;
        G = (groups + per - 1) / per;
        if (tiles * G > INT32_MAX) return hipErrorInvalidValue;   // grid size
        hipLaunchKernelGGL((step16_kernel<DISC, KS>), dim3(static_cast<unsigned>(tiles * G)),
                           dim3(kWave), 0, st, a);
    } else {
        hipLaunchKernelGGL((step_kernel<DISC, KS>), dim3(grid), dim3(kWave), 0, st, a);
    }
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
