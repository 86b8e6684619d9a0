// scan_bwd_kernel.hip -- backward pass of the selective scan and its gate for
// gfx950.
//
// Computes the reverse-time adjoint of mamba1CpuBackward (builderforce-memory-
// engine 2026.7.12 -> 2026.9.27, src/training/mamba1_cpu.ts: its gate,
// reverse-time scan, A_log clamp mask and softplus parts): per
// (b, d) column, with dY = dout SiLU(z), g_n the adjoint carried from step
// t+1 and dh_n = C_n dY + g_n,
//   du = D dY + sum_n dh_n bBar_n            g_n <- dh_n aBar_n
//   ddv = sum_n aBar_n (dh_n h_{t-1,n} A_n + dh_n u dbBar_n/ddv / aBar_n)
//   dA_n += dv aBar_n dh_n h_{t-1,n} + dh_n u dbBar_n/dA
//   dB[r,n] = sum_d dh_n u dbBar_n/dB          dC[r,n] = sum_d dY h_t,n
//   dz = dout y SiLU'(z),  ddelta = ddv sigmoid(delta),  dD = sum dY u
//
// Mapping.  A channel tile is (batch row, 32 channels); lane (half, q) owns
// channel q of the tile and the 8 states n = 8 half + j, so the per-lane
// state vectors (h, adjoint, dA) stay at 8 registers each and the two halves
// of a channel combine their sums with one cross-half add.  The flattened
// (tile, t) space is cut into equal segments, one wave each, so that all
// wave slots carry the same work; a segment that crosses the end of a tile
// is worked as one piece per tile.
//
// Work per piece [t0, t1) of a tile:
//   1. h(t0-1) by decay-bounded forward replay (as in the forward kernel).
//   2. Forward over the segment, storing h at every 8-step block start in the
//      checkpoint workspace (2 KB per block).
//   (1 and 2 are skipped when the forward pass's own states at every 8th
//   step are given: the blocks then start from those.)
//   3. The adjoint carried into t1-1 by decay-bounded reverse replay: walk
//      delta forward from t1 until every lane's slowest state has decayed by
//      2^-c (c = MSS_REPLAY_DECAY_BITS), then run the adjoint recurrence
//      backwards from there with g = 0.
//   4. Blocks in reverse order: reload the block's checkpoint, recompute its
//      8 states into registers (emitting dz and the dC terms on the way),
//      then run the adjoint through the block (emitting du, ddelta and the dB
//      terms).
// Cross-channel sums: each step's 8 dB (or dC) values per lane are reduced
// over the 32 channels of the tile with a transpose-reduce (one exchange
// level per lane bit: row swap, DPP), then written per tile to a
// partial buffer that a second kernel sums over tiles in a fixed order; dA
// and dD are written per piece and summed the same way.  No atomics: the
// result is bitwise reproducible.
#include "device_math.h"
#include "launch_bwd.h"

namespace mss {
namespace {

constexpr int kT = 8;                          // steps per block
constexpr int kH = 8;                          // states per lane
constexpr int kBackBlk = 16;
constexpr float kDecayCut = MSS_REPLAY_DECAY_BITS;
constexpr float kSmallX = 0.015625f;           // expm1 cubic below |dv A| = 2^-6
constexpr float kSmallX2 = kSmallX * kLog2e;
constexpr int kNone = 0, kFirst = 1, kAll = 2;  // which states take the accurate path

struct BwdCols {
    const float* __restrict__ u;
    const float* __restrict__ delta;
    const float* __restrict__ A_log;
    const float* __restrict__ Bm;
    const float* __restrict__ Cm;
    const float* __restrict__ Dv;
    const float* __restrict__ z;
    const float* __restrict__ h0;
    const float* __restrict__ hck;    // (B, ceil(L/8), D, N) or null
    const float* __restrict__ dout;
    float* __restrict__ du;
    float* __restrict__ ddelta;
    float* __restrict__ dz;
    float* __restrict__ dh0;
    float* __restrict__ ckpt;     // (waves, blocks per segment, 2, 64, 4)
    float* __restrict__ partB;    // (B, tiles, L, 16)
    float* __restrict__ partC;    // (B, tiles, L, 16)
    float* __restrict__ partA;    // (waves, 64, 8)
    float* __restrict__ partD;    // (waves, 32)
};

__device__ __forceinline__ float as_f(int v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ int as_i(float v) { return __builtin_bit_cast(int, v); }
__device__ __forceinline__ uint32_t as_u(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float u_as_f(uint32_t v) { return __builtin_bit_cast(float, v); }

// Lane exchanges inside a 32-lane half.
__device__ __forceinline__ float xor8(float v) {    // DPP row_ror:8 (rotation by 8 in 16 lanes)
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), 0x128, 0xf, 0xf, true));
}
__device__ __forceinline__ float xor7(float v) {    // DPP row_half_mirror (lane i <-> 7 - i)
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), 0x141, 0xf, 0xf, true));
}
__device__ __forceinline__ float xor2(float v) {    // DPP quad_perm [2,3,0,1]
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), 0x4e, 0xf, 0xf, true));
}
__device__ __forceinline__ float xor1(float v) {    // DPP quad_perm [1,0,3,2]
    return as_f(__builtin_amdgcn_mov_dpp(as_i(v), 0xb1, 0xf, 0xf, true));
}

// gfx950's v_permlane16_swap trades the odd 16-lane rows of its first
// operand for the even rows of its second.  With x, y in every lane this
// leaves x's rows (0, 0, 2, 2) and y's rows (1, 1, 3, 3) behind, so the sum
// of the two results is, in lanes with bit 4 clear, x plus x of lane + 16,
// and in lanes with bit 4 set, y plus y of lane - 16 (lower lane first in
// both).  (Both results are copied out before use.)
__device__ __forceinline__ float swap16_sum(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(as_u(x), as_u(y), false, false);
    const uint32_t nx = r[0], ny = r[1];
    return u_as_f(nx) + u_as_f(ny);
}

// Sum of the two halves of a channel (lanes l and l ^ 32): v_permlane32_swap
// of v with itself leaves the lower half of v in both halves of one result
// and the upper half in both halves of the other.
__device__ __forceinline__ float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u(v), as_u(v), false, false);
    const uint32_t lo = r[0], hi = r[1];
    return u_as_f(lo) + u_as_f(hi);
}

// The channel sums of two values at once: the swap of a with b leaves
// (a, b) of the lower half in one result and (a, b) of the upper half in the
// other, so lanes 0-31 get a_l + a_{l+32} and lanes 32-63 b_{l-32} + b_l.
__device__ __forceinline__ float pair_sum2(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
    const uint32_t lo = r[0], hi = r[1];
    return u_as_f(lo) + u_as_f(hi);
}

// Sum over the 32 lanes of this half of v[j], for j = 4 b3 + 2 b4 + b2
// (b4, b3, b2: bits 4, 3, 2 of the lane): three exchange levels that each
// keep half of the values and add the partner's other half -- lane bit 4
// with register bit 1 (the row swap above), lane bit 3 with register bit 2,
// lane bit 2 with register bit 0 -- then two plain levels.
__device__ __forceinline__ float reduce8(const float (&v)[kH]) {
    const uint32_t q = threadIdx.x & 31u;
    const bool b3 = q & 8u, b2 = q & 4u;
    float w4[4];   // w4[2 r2 + r0]: register 4 r2 + 2 b4 + r0
#pragma unroll
    for (int r2 = 0; r2 < 2; r2++)
#pragma unroll
        for (int r0 = 0; r0 < 2; r0++)
            w4[2 * r2 + r0] = swap16_sum(v[4 * r2 + r0], v[4 * r2 + 2 + r0]);
    float w2[2];   // w2[r0]: register 4 b3 + 2 b4 + r0
#pragma unroll
    for (int r0 = 0; r0 < 2; r0++) {
        const float keep = b3 ? w4[2 + r0] : w4[r0];
        const float send = b3 ? w4[r0] : w4[2 + r0];
        w2[r0] = keep + xor8(send);
    }
    const float keep = b2 ? w2[1] : w2[0];
    const float send = b2 ? w2[0] : w2[1];
    float w1 = keep + xor7(send);
    w1 += xor2(w1);
    w1 += xor1(w1);
    return w1;
}

// State (within the lane's half) whose sum reduce8 leaves in this lane.
__device__ __forceinline__ uint32_t reduce8_state() {
    const uint32_t q = threadIdx.x & 31u;
    return ((q >> 1) & 4u) | ((q >> 3) & 2u) | ((q >> 2) & 1u);
}

// sigmoid(v); SiLU(v) = v sigmoid(v) and d SiLU / dv = s (1 + v (1 - s)) with
// s = sigmoid(v) are formed from it where used.
__device__ __forceinline__ float sigmoid(float v) { return rcp(1.0f + ex2(-kLog2e * v)); }

// expm1(x) for |x| < 2^-6 (relative truncation < 2e-7) else a - 1.
__device__ __forceinline__ float em1_of(float x, float a) {
    const float p = x * __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 6.0f, 0.5f), 1.0f);
    return __builtin_fabsf(x) < kSmallX ? p : a - 1.0f;
}

template <int DISC, int NS>
struct Bwd {
    static constexpr bool kZoh = DISC == MSS_DISC_ZOH;

    const BwdCols& c;
    const int64_t L, D;
    const int N;
    const int64_t b;
    const uint32_t d;          // channel, clamped to D - 1
    const bool live;           // the lane's channel exists
    const uint32_t half;
    const bool gated;
    float4* lds;               // 8 steps: B rows [0, 32), C rows [32, 64) (16 floats per row)
    float4* acache;            // aBar of a block's 8 steps: [step][half][lane] (8 floats per lane)

    float A2[kH], Ai[kH], An[kH];
    float min_a2, dvec;

    __device__ Bwd(const BwdCols& c_, const BwdShape& s, int64_t b_, int64_t d_raw, float4* lds_)
        : c(c_), L(s.L), D(s.D), N(NS > 0 ? NS : s.N), b(b_),
          d(static_cast<uint32_t>(d_raw < s.D ? d_raw : s.D - 1)), live(d_raw < s.D),
          half(threadIdx.x >> 5), gated(c_.z != nullptr), lds(lds_), acache(lds_ + kWave) {}

    __device__ __forceinline__ bool valid(int j) const {
        return NS > 0 || static_cast<int>(half) * kH + j < N;
    }
    __device__ __forceinline__ int64_t row(int64_t t) const { return b * L + t; }
    __device__ __forceinline__ float ld(const float* base, int64_t t) const {
        return base[row(t) * D + d];
    }

    __device__ __forceinline__ void init() {
        float mn = 3.0e38f;
#pragma unroll
        for (int j = 0; j < kH; j++) {
            if (valid(j)) {
                const float A = a_cont(c.A_log[d * N + half * kH + j]);
                An[j] = A;
                A2[j] = A * kLog2e;
                Ai[j] = 1.0f / A;
                mn = __builtin_fminf(mn, -A2[j]);
            } else {
                An[j] = -1.0f;
                A2[j] = -kLog2e;
                Ai[j] = -1.0f;
            }
        }
        min_a2 = mn;
        dvec = c.Dv ? c.Dv[d] : 0.0f;
    }

    // B and C rows of steps t0 .. t0+7 into LDS, zero-padded to 16 states
    // (rows past the sequence end repeat its last row and are never used).
    __device__ __forceinline__ void stage(int64_t t0) const {
        const uint32_t lane = threadIdx.x;
        const uint32_t q = lane & 31u;
        int64_t t = t0 + (q >> 2);
        t = t < L ? t : L - 1;
        const float* base = (lane < 32 ? c.Bm : c.Cm) + row(t) * N;
        const int col = static_cast<int>(q & 3u) * 4;
        float4 v;
        if constexpr (NS == 16) {
            v = *reinterpret_cast<const float4*>(base + col);
        } else {
            v.x = col + 0 < N ? base[col + 0] : 0.0f;
            v.y = col + 1 < N ? base[col + 1] : 0.0f;
            v.z = col + 2 < N ? base[col + 2] : 0.0f;
            v.w = col + 3 < N ? base[col + 3] : 0.0f;
        }
        __builtin_amdgcn_wave_barrier();
        lds[lane] = v;
        __builtin_amdgcn_wave_barrier();
    }
    __device__ __forceinline__ void read_row(int base, int i, float (&v)[kH]) const {
        const float4 p = lds[base + i * 4 + 2 * half];
        const float4 q = lds[base + i * 4 + 2 * half + 1];
        v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
        v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
    }

    // ---- forward state update (as the forward kernel) -------------------
    // SLOW: the decay is applied as h + m h with m = expm1(dv A) accurate
    // (cubic below |dv A| = 2^-6), since fl(aBar) next to 1 carries an
    // absolute error that would compound over a long memory.
    template <bool SLOW>
    __device__ __forceinline__ void fwd_state(int j, float& h, float uv, float dv, float dvu,
                                              float Bj, float& aout) const {
        const float x2 = dv * A2[j];
        const float a = ex2(x2);
        aout = a;
        if constexpr (!SLOW) {
            if constexpr (kZoh) {
                const float k = (uv * Ai[j]) * Bj;
                h = __builtin_fmaf(a, h + k, -k);
            } else {
                h = __builtin_fmaf(a, h, dvu * Bj);
            }
        } else {
            const float m = em1_of(x2 * kLn2, a);
            if constexpr (kZoh) {
                const float k = (uv * Ai[j]) * Bj;
                h = __builtin_fmaf(m, h + k, h);
            } else {
                h = __builtin_fmaf(dvu, Bj, __builtin_fmaf(m, h, h));
            }
        }
    }

    // SM (slow mode of the block, see slow_mode): kNone, kFirst (state 0
    // takes the accurate path) or kAll.
    template <int SM>
    static constexpr bool slow_state(int j) {
        return SM == kAll || (SM == kFirst && j == 0);
    }

    // av: the step's aBar per state (0 for padding states).
    template <int SM>
    __device__ __forceinline__ void fwd(float (&h)[kH], float uv, float dv, const float (&Bv)[kH],
                                        float (&av)[kH]) const {
        fwd<SM>(h, h, uv, dv, Bv, av);
    }
    // The same from hin into hout (hin is left as it was).
    template <int SM>
    __device__ __forceinline__ void fwd(const float (&hin)[kH], float (&hout)[kH], float uv,
                                        float dv, const float (&Bv)[kH], float (&av)[kH]) const {
        const float dvu = dv * uv;
#pragma unroll
        for (int j = 0; j < kH; j++) {
            av[j] = 0.0f;
            float hv = hin[j];
            if (valid(j)) {
                if (slow_state<SM>(j))
                    fwd_state<true>(j, hv, uv, dv, dvu, Bv[j], av[j]);
                else
                    fwd_state<false>(j, hv, uv, dv, dvu, Bv[j], av[j]);
            }
            hout[j] = hv;
        }
    }

    // ---- reverse (adjoint) step ------------------------------------------
    // FULL: also the gradient terms (du, ddv, dA, dB); otherwise only g.
    // du_acc and ddv_acc are this lane's sums over its states for the step.
    // With dh = C dY + g and gn = aBar dh (the adjoint passed to step t-1):
    //   ZOH (q = (aBar-1)/A, K = u B / A):
    //     du += dh q B,  dB term = dh q u,  ddv += gn (h_{t-1} A + u B),
    //     dA += dh (dv aBar (h_{t-1} + K) - K q)
    //   EULER: du += dh dv B,  dB term = dh u dv,
    //     ddv += gn h_{t-1} A + dh u B,  dA += gn dv h_{t-1}
    // SLOW (some lane has |dv A| < 2^-6): m = aBar - 1 from its cubic, gn as
    // dh + m dh, and for ZOH the dA term as dv aBar h_{t-1} + K t5 with
    // t5 = dv aBar - q from its series dv x (1/2 + x/3 + x^2/8 + x^3/30)
    // (x = dv A) where |x| < 2^-6: the direct difference cancels there.
    // FULL steps take aBar from the block's recompute (a_in); the replay
    // computes it.
    template <bool SLOW, bool FULL>
    __device__ __forceinline__ void rev_state(int j, float& g, float& dA, float hp, float uv, float dv, float udv, float dY, float Bj,
                                              float Cj, float a_in, float& du_acc,
                                              float& ddv_acc, float& dBp) const {
        const float x2 = (SLOW || !FULL) ? dv * A2[j] : 0.0f;
        const float a = FULL ? a_in : ex2(x2);
        const float dh = __builtin_fmaf(Cj, dY, g);
        float m = 0.0f, gn;
        if constexpr (SLOW) {
            m = em1_of(x2 * kLn2, a);
            gn = __builtin_fmaf(m, dh, dh);
        } else {
            gn = dh * a;
        }
        g = gn;
        if constexpr (FULL) {
            if constexpr (kZoh) {
                // q = (aBar - 1) / A: one fma on the fast path, where
                // |dv A| >= 2^-6 keeps aBar - 1 away from cancellation
                float q;
                if constexpr (!SLOW) q = __builtin_fmaf(a, Ai[j], -Ai[j]);
                else q = m * Ai[j];
                const float dq = dh * q;
                du_acc = __builtin_fmaf(dq, Bj, du_acc);
                dBp = dq * uv;
                const float uB = uv * Bj;
                const float K = uB * Ai[j];
                if constexpr (!SLOW) {
                    // with X = gn (h_{t-1} + K) = dh aBar (h_{t-1} + K) the
                    // ddv term gn (h_{t-1} A + u B) is A X and the dA term
                    // dv X - dh q K
                    const float X = gn * (hp + K);
                    ddv_acc = __builtin_fmaf(X, An[j], ddv_acc);
                    dA = __builtin_fmaf(-dq, K, __builtin_fmaf(dv, X, dA));
                } else {
                    ddv_acc = __builtin_fmaf(gn, __builtin_fmaf(hp, An[j], uB), ddv_acc);
                    const float x = x2 * kLn2;
                    const float ph = __builtin_fmaf(
                        x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 30.0f, 0.125f), 1.0f / 3.0f),
                        0.5f);
                    const float t5d = __builtin_fmaf(dv, a, -q);
                    const float t5 = __builtin_fabsf(x) < kSmallX ? (dv * x) * ph : t5d;
                    dA = __builtin_fmaf(dh, __builtin_fmaf(dv * a, hp, K * t5), dA);
                }
            } else {
                // du_acc collects sum_n dh B here; rev scales it by dv (du)
                // and by u (its ddv part) after the last state
                du_acc = __builtin_fmaf(dh, Bj, du_acc);
                dBp = dh * udv;
                const float gh = gn * hp;
                ddv_acc = __builtin_fmaf(gh, An[j], ddv_acc);
                dA = __builtin_fmaf(gh, dv, dA);
            }
        }
    }

    // hp: the states before the step.
    template <int SM, bool FULL>
    __device__ __forceinline__ void rev(float (&g)[kH], float (&dA)[kH], const float (&hp)[kH],
                                        float uv, float dv, float dY,
                                        const float (&Bv)[kH], const float (&Cv)[kH],
                                        const float (&av)[kH], float& du_acc, float& ddv_acc,
                                        float (&dBp)[kH]) const {
        const float udv = uv * dv;
#pragma unroll
        for (int j = 0; j < kH; j++) {
            if (!valid(j)) {
                if constexpr (FULL) dBp[j] = 0.0f;
                continue;
            }
            if (slow_state<SM>(j))
                rev_state<true, FULL>(j, g[j], dA[j], hp[j], uv, dv, udv, dY, Bv[j],
                                      Cv[j], av[j], du_acc, ddv_acc, dBp[j]);
            else
                rev_state<false, FULL>(j, g[j], dA[j], hp[j], uv, dv, udv, dY, Bv[j],
                                       Cv[j], av[j], du_acc, ddv_acc, dBp[j]);
        }
        if constexpr (FULL && !kZoh) {
            ddv_acc = __builtin_fmaf(uv, du_acc, ddv_acc);
            du_acc *= dv;
        }
    }

    // ---- decay-bounded replay bounds --------------------------------------
    __device__ __forceinline__ int64_t replay_start(int64_t t0) const {
        if (t0 == 0) return 0;
        float S = 0.0f;
        int64_t t = t0;
        while (true) {
            float dd[kBackBlk];
#pragma unroll
            for (int i = 0; i < kBackBlk; i++) {
                const int64_t tt = t - 1 - i;
                dd[i] = ld(c.delta, tt >= 0 ? tt : 0);
            }
#pragma unroll
            for (int i = 0; i < kBackBlk; i++) {
                const int64_t tt = t - 1 - i;
                if (tt < 0) return 0;
                S += softplus(dd[i]);
                if (wave_all(S * min_a2 >= kDecayCut)) return tt;
            }
            t -= kBackBlk;
        }
    }

    // End (exclusive) of the reverse replay that carries the adjoint into t1-1.
    __device__ __forceinline__ int64_t replay_end(int64_t t1) const {
        if (t1 >= L) return L;
        float S = 0.0f;
        int64_t t = t1;
        while (true) {
            float dd[kBackBlk];
#pragma unroll
            for (int i = 0; i < kBackBlk; i++) {
                const int64_t tt = t + i;
                dd[i] = ld(c.delta, tt < L ? tt : L - 1);
            }
#pragma unroll
            for (int i = 0; i < kBackBlk; i++) {
                const int64_t tt = t + i;
                if (tt >= L) return L;
                S += softplus(dd[i]);
                if (wave_all(S * min_a2 >= kDecayCut)) return tt + 1;
            }
            t += kBackBlk;
        }
    }

    // A state needs the accurate path in a block when some lane has
    // |dv A| < 2^-6 at some step of it.  The block then runs kNone (no such
    // state), kFirst (only state 0: with A ordered by magnitude, as in the
    // S4D initialisation, state 0 holds the slowest mode) or kAll.
    __device__ __forceinline__ int slow_mode(const float (&dv)[kT], int n) const {
        float mn = 3.0e38f;
#pragma unroll
        for (int i = 0; i < kT; i++) mn = i < n ? __builtin_fminf(mn, dv[i]) : mn;
        bool rest = false;
#pragma unroll
        for (int j = 1; j < kH; j++)
            if (valid(j)) rest = rest || (mn * -A2[j] < kSmallX2);
        if (wave_any(rest)) return kAll;
        return wave_any(mn * -A2[0] < kSmallX2) ? kFirst : kNone;
    }

    // ---- forward sweep over [ta, tb) in blocks of 8 from ta ---------------
    // CKPT: store h at every block start to ck (2 KB per block: states 0-3
    // of the 64 lanes, then states 4-7, so each store is one contiguous 1 KB).
    template <bool CKPT>
    __device__ __forceinline__ void fwd_sweep(float (&h)[kH], int64_t ta, int64_t tb, float* ck) const {
        for (int64_t s = ta; s < tb; s += kT) {
            const int n = tb - s < kT ? static_cast<int>(tb - s) : kT;
            if constexpr (CKPT) {
                float4* p = reinterpret_cast<float4*>(ck) + threadIdx.x;
                p[0] = make_float4(h[0], h[1], h[2], h[3]);
                p[kWave] = make_float4(h[4], h[5], h[6], h[7]);
                ck += kWave * kH;
            }
            float uu[kT], dv[kT];
#pragma unroll
            for (int i = 0; i < kT; i++) {
                const int64_t t = s + i < L ? s + i : L - 1;
                uu[i] = ld(c.u, t);
                dv[i] = ld(c.delta, t);
            }
            stage(s);
#pragma unroll
            for (int i = 0; i < kT; i++) dv[i] = softplus(dv[i]);
            const int sm = slow_mode(dv, n);
            if (sm == kNone)
                fwd_block<kNone>(h, uu, dv, n);
            else if (sm == kFirst)
                fwd_block<kFirst>(h, uu, dv, n);
            else
                fwd_block<kAll>(h, uu, dv, n);
        }
    }

    // dY of step t (0 for lanes without a channel).
    __device__ __forceinline__ float grad_y(float go, float zv) const {
        const float v = gated ? go * silu(zv) : go;
        return live ? v : 0.0f;
    }

    template <int SM>
    __device__ __forceinline__ void fwd_block(float (&h)[kH], const float (&uu)[kT],
                                              const float (&dv)[kT], int n) const {
#pragma unroll
        for (int i = 0; i < kT; i++) {
            if (i >= n) break;
            float Bv[kH], av[kH];
            read_row(0, i, Bv);
            fwd<SM>(h, uu[i], dv[i], Bv, av);
        }
    }

    // Only g is updated; the gradient arguments of rev are not read.
    template <int SM>
    __device__ __forceinline__ void rev_block(float (&g)[kH], const float (&dv)[kT],
                                              const float (&dY)[kT], int n) const {
        float dA[kH] = {}, hp[kH] = {}, dBp[kH], Bv[kH] = {}, av[kH] = {}, du_acc = 0.0f,
              ddv_acc = 0.0f;
#pragma unroll
        for (int i = kT - 1; i >= 0; i--) {
            if (i >= n) continue;
            float Cv[kH];
            read_row(32, i, Cv);
            rev<SM, false>(g, dA, hp, 0.0f, dv[i], dY[i], Bv, Cv, av, du_acc, ddv_acc, dBp);
        }
    }

    // ---- reverse replay over [ta, tb), adjoint only -----------------------
    __device__ __forceinline__ void rev_sweep(float (&g)[kH], int64_t ta, int64_t tb) const {
        const int64_t nb = (tb - ta + kT - 1) / kT;
        for (int64_t k = nb - 1; k >= 0; k--) {
            const int64_t s = ta + k * kT;
            const int n = tb - s < kT ? static_cast<int>(tb - s) : kT;
            float dv[kT], dY[kT];
#pragma unroll
            for (int i = 0; i < kT; i++) {
                const int64_t t = s + i < L ? s + i : L - 1;
                dv[i] = ld(c.delta, t);
                const float go = ld(c.dout, t);
                const float zv = gated ? ld(c.z, t) : 0.0f;
                dY[i] = grad_y(go, zv);
            }
            stage(s);
#pragma unroll
            for (int i = 0; i < kT; i++) dv[i] = softplus(dv[i]);
            const int sm = slow_mode(dv, n);
            if (sm == kNone)
                rev_block<kNone>(g, dv, dY, n);
            else if (sm == kFirst)
                rev_block<kFirst>(g, dv, dY, n);
            else
                rev_block<kAll>(g, dv, dY, n);
        }
    }

    // ---- one block of the main pass ---------------------------------------
    template <int SM>
    __device__ __forceinline__ void block(float (&g)[kH], float (&dA)[kH], float& dD,
                                          const float (&h_in)[kH], int64_t s, int n,
                                          const float (&uu)[kT], const float (&dl)[kT],
                                          const float (&dv)[kT], const float (&go)[kT],
                                          const float (&zz)[kT], float* pB, float* pC) const {
        float hist[kT + 1][kH];   // hist[i]: the states before step i of the block
        float dY[kT];
#pragma unroll
        for (int j = 0; j < kH; j++) hist[0][j] = h_in[j];
        const bool writer = live && half == 0;
        const bool red_writer = (threadIdx.x & 3u) == 0;
        const uint32_t n_out = half * kH + reduce8_state();
        // Recompute the block's states (forward), with dz and the dC terms.
#pragma unroll
        for (int i = 0; i < kT; i++) {
            if (i >= n) break;
            float Bv[kH], Cv[kH], av[kH];
            read_row(0, i, Bv);
            read_row(32, i, Cv);
            fwd<SM>(hist[i], hist[i + 1], uu[i], dv[i], Bv, av);
            const float (&h)[kH] = hist[i + 1];
            // aBar of the step, kept for the adjoint below (this lane only)
            acache[(i * 2) * kWave + threadIdx.x] = make_float4(av[0], av[1], av[2], av[3]);
            acache[(i * 2 + 1) * kWave + threadIdx.x] = make_float4(av[4], av[5], av[6], av[7]);
            float yp = 0.0f;
#pragma unroll
            for (int j = 0; j < kH; j++) yp = __builtin_fmaf(Cv[j], h[j], yp);
            const float y = __builtin_fmaf(dvec, uu[i], pair_sum(yp));
            // sigmoid(z) once for dY = dout SiLU(z) and for dz
            const float sz = gated ? sigmoid(zz[i]) : 0.0f;
            dY[i] = live ? (gated ? go[i] * (zz[i] * sz) : go[i]) : 0.0f;
            const int64_t r = row(s + i);
            if (gated && writer)
                c.dz[r * D + d] = go[i] * y * (sz * __builtin_fmaf(zz[i], 1.0f - sz, 1.0f));
            float dCp[kH];
#pragma unroll
            for (int j = 0; j < kH; j++) dCp[j] = dY[i] * h[j];
            const float sC = reduce8(dCp);
            if (red_writer) pC[(s + i) * 16 + n_out] = sC;
        }
        // Adjoint through the block, newest step first.
#pragma unroll
        for (int i = kT - 1; i >= 0; i--) {
            if (i >= n) continue;
            float Bv[kH], Cv[kH], dBp[kH];
            read_row(0, i, Bv);
            read_row(32, i, Cv);
            const float4 a_lo = acache[(i * 2) * kWave + threadIdx.x];
            const float4 a_hi = acache[(i * 2 + 1) * kWave + threadIdx.x];
            const float av[kH] = {a_lo.x, a_lo.y, a_lo.z, a_lo.w, a_hi.x, a_hi.y, a_hi.z, a_hi.w};
            float du_acc = 0.0f, ddv_acc = 0.0f;
            rev<SM, true>(g, dA, hist[i], uu[i], dv[i], dY[i], Bv, Cv, av, du_acc, ddv_acc, dBp);
            // the lower half stores du, the upper half ddelta (same channel)
            const float sum = pair_sum2(du_acc, ddv_acc);
            const float val = half == 0 ? __builtin_fmaf(dY[i], dvec, sum) : sum * sigmoid(dl[i]);
            float* dst = half == 0 ? c.du : c.ddelta;
            if (live) dst[row(s + i) * D + d] = val;
            dD = __builtin_fmaf(dY[i], uu[i], dD);
            const float sB = reduce8(dBp);
            if (red_writer) pB[(s + i) * 16 + n_out] = sB;
        }
    }
};

// One piece [t0, t1) of channel tile ti (batch row b = ti / tiles_per_b);
// slot: the piece's index among the pieces of tile ti, which selects its
// rows of partA and partD; ck: this wave's checkpoint area.
template <int DISC, int NS>
__device__ __forceinline__ void bwd_piece(const BwdCols& c, const BwdShape& s, int64_t ti,
                                          int64_t t0, int64_t t1, int64_t slot, float* ck,
                                          float4* lds) {
    const int64_t b = ti / s.tiles_per_b;
    const int64_t ct = ti - b * s.tiles_per_b;
    const uint32_t lane = threadIdx.x;

    Bwd<DISC, NS> bw(c, s, b, ct * 32 + (lane & 31u), lds);
    bw.init();

    if (!c.hck) {
        // 1. h(t0 - 1)
        float h[kH];
        const int64_t tw = bw.replay_start(t0);
#pragma unroll
        for (int j = 0; j < kH; j++)
            h[j] = (tw == 0 && c.h0 && bw.valid(j))
                       ? c.h0[(b * s.D + bw.d) * bw.N + bw.half * kH + j]
                       : 0.0f;
        bw.template fwd_sweep<false>(h, tw, t0, nullptr);

        // 2. checkpoints of the piece
        bw.template fwd_sweep<true>(h, t0, t1, ck);
        // The checkpoints are read back by this wave below.
        __threadfence_block();
    }
    // (with the forward's checkpoints, every block below starts from them:
    // t0 is a multiple of 8, so the blocks of the piece are the 8-step
    // blocks of the checkpoints)
    const int64_t nck = (s.L + 7) >> 3;

    // 3. adjoint carried into t1 - 1
    float g[kH];
#pragma unroll
    for (int j = 0; j < kH; j++) g[j] = 0.0f;
    bw.rev_sweep(g, t1, bw.replay_end(t1));

    // 4. blocks of the piece, newest first
    float dA[kH];
#pragma unroll
    for (int j = 0; j < kH; j++) dA[j] = 0.0f;
    float dD = 0.0f;
    float* pB = c.partB + ti * s.L * 16;
    float* pC = c.partC + ti * s.L * 16;
    const int64_t nb = (t1 - t0 + kT - 1) / kT;
    for (int64_t k = nb - 1; k >= 0; k--) {
        const int64_t st = t0 + k * kT;
        const int n = t1 - st < kT ? static_cast<int>(t1 - st) : kT;
        float uu[kT], dl[kT], dv[kT], go[kT], zz[kT];
#pragma unroll
        for (int i = 0; i < kT; i++) {
            const int64_t t = st + i < s.L ? st + i : s.L - 1;
            uu[i] = bw.ld(c.u, t);
            dl[i] = bw.ld(c.delta, t);
            go[i] = bw.ld(c.dout, t);
            zz[i] = c.z ? bw.ld(c.z, t) : 0.0f;
        }
        float hin[kH];
        if (c.hck) {
            // this lane's 8 states of the block's start: a channel's 16
            // states are 64 contiguous bytes, the tile's 32 channels 2 KB
            const float* p = c.hck + ((b * nck + (st >> 3)) * s.D + bw.d) * bw.N + bw.half * kH;
            if constexpr (NS == 16) {
                const float4 lo = reinterpret_cast<const float4*>(p)[0];
                const float4 hi = reinterpret_cast<const float4*>(p)[1];
                hin[0] = lo.x; hin[1] = lo.y; hin[2] = lo.z; hin[3] = lo.w;
                hin[4] = hi.x; hin[5] = hi.y; hin[6] = hi.z; hin[7] = hi.w;
            } else {
#pragma unroll
                for (int j = 0; j < kH; j++) hin[j] = bw.valid(j) ? p[j] : 0.0f;
            }
        } else {
            const float4* p = reinterpret_cast<const float4*>(ck + k * (kWave * kH)) + lane;
            const float4 h_lo = p[0], h_hi = p[kWave];
            hin[0] = h_lo.x; hin[1] = h_lo.y; hin[2] = h_lo.z; hin[3] = h_lo.w;
            hin[4] = h_hi.x; hin[5] = h_hi.y; hin[6] = h_hi.z; hin[7] = h_hi.w;
        }
        bw.stage(st);
#pragma unroll
        for (int i = 0; i < kT; i++) dv[i] = softplus(dl[i]);
        const int sm = bw.slow_mode(dv, n);
        if (sm == kNone)
            bw.template block<kNone>(g, dA, dD, hin, st, n, uu, dl, dv, go, zz, pB, pC);
        else if (sm == kFirst)
            bw.template block<kFirst>(g, dA, dD, hin, st, n, uu, dl, dv, go, zz, pB, pC);
        else
            bw.template block<kAll>(g, dA, dD, hin, st, n, uu, dl, dv, go, zz, pB, pC);
    }

    // 5. the piece's partial sums and dh0
    const int64_t row = ti * s.pieces + slot;
    float4* pa = reinterpret_cast<float4*>(c.partA + (row * kWave + lane) * kH);
    pa[0] = make_float4(dA[0], dA[1], dA[2], dA[3]);
    pa[1] = make_float4(dA[4], dA[5], dA[6], dA[7]);
    if (lane < 32) c.partD[row * 32 + lane] = dD;
    if (t0 == 0 && c.dh0 && bw.live) {
#pragma unroll
        for (int j = 0; j < kH; j++)
            if (bw.valid(j)) c.dh0[(b * s.D + bw.d) * bw.N + bw.half * kH + j] = g[j];
    }
}

// Wave w takes steps [w seg, (w+1) seg) of the flattened (tile, t) space,
// so every wave has the same number of steps; a range that crosses the end
// of a tile is taken as one piece per tile, one after the other.
template <int DISC, int NS>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void scan_bwd_kernel(
    BwdCols c, BwdShape s) {
    __shared__ float4 lds[kWave + kT * kWave * 2];   // B/C staging, then the aBar cache
    const int64_t w = blockIdx.x;
    const int64_t g0 = w * s.seg;
    const int64_t g1 = g0 + s.seg < s.total ? g0 + s.seg : s.total;
    float* ck = c.ckpt + w * s.blocks_per_seg * (kWave * kH);
    for (int64_t g = g0; g < g1;) {
        const int64_t ti = g / s.Lp;
        const int64_t t0 = g - ti * s.Lp;
        if (t0 >= s.L) {        // the tile's padding steps
            g = (ti + 1) * s.Lp;
            continue;
        }
        const int64_t t1 = t0 + (g1 - g) < s.L ? t0 + (g1 - g) : s.L;
        const int64_t slot = w - (ti * s.Lp) / s.seg;   // waves before w that cover tile ti
        bwd_piece<DISC, NS>(c, s, ti, t0, t1, slot, ck, lds);
        g += t1 - t0;
    }
}

// Number of pieces of tile ti (one per wave whose step range meets it).
__device__ __forceinline__ int64_t tile_pieces(const BwdShape& s, int64_t ti) {
    return (ti * s.Lp + s.L - 1) / s.seg - (ti * s.Lp) / s.seg + 1;
}

// Cross-tile and cross-piece sums, fixed order:
//   dB[r, n], dC[r, n] = sum over channel tiles of the partial rows;
//   dA_log[d, n] = A[d, n] * sum over (b, piece) (0 outside the clamp);
//   dD[d] = sum over (b, piece).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdCols c, BwdShape s, float* dB,
                                                         float* dC, float* dA_log, float* dD) {
    const int64_t M = s.B * s.L;
    // dB/dC items: four states (one 16-byte piece of a row) each when N = 16,
    // else one state each
    const bool vec = s.N == 16;
    const int64_t nBC = vec ? M * 4 : M * s.N;
    const int64_t nA = s.D * s.N;
    const int64_t total = nBC + nA + (dD ? s.D : 0);
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        if (i < nBC && vec) {
            const int64_t r = i >> 2, n0 = (i & 3) * 4;
            const int64_t b = r / s.L, t = r - b * s.L;
            float4 sb = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sc = sb;
            for (int64_t ct = 0; ct < s.tiles_per_b; ct++) {
                const int64_t o = ((b * s.tiles_per_b + ct) * s.L + t) * 16 + n0;
                const float4 pb = *reinterpret_cast<const float4*>(c.partB + o);
                const float4 pc = *reinterpret_cast<const float4*>(c.partC + o);
                sb.x += pb.x; sb.y += pb.y; sb.z += pb.z; sb.w += pb.w;
                sc.x += pc.x; sc.y += pc.y; sc.z += pc.z; sc.w += pc.w;
            }
            *reinterpret_cast<float4*>(dB + r * 16 + n0) = sb;
            *reinterpret_cast<float4*>(dC + r * 16 + n0) = sc;
        } else if (i < nBC) {
            const int64_t r = i / s.N, n = i - r * s.N;
            const int64_t b = r / s.L, t = r - b * s.L;
            float sb = 0.0f, sc = 0.0f;
            for (int64_t ct = 0; ct < s.tiles_per_b; ct++) {
                const int64_t o = ((b * s.tiles_per_b + ct) * s.L + t) * 16 + n;
                sb += c.partB[o];
                sc += c.partC[o];
            }
            dB[i] = sb;
            dC[i] = sc;
        } else if (i < nBC + nA) {
            const int64_t e = i - nBC;
            const int64_t d = e / s.N, n = e - d * s.N;
            const int64_t ct = d / 32, q = d - ct * 32;
            const int64_t lane = (n / kH) * 32 + q, j = n % kH;
            float acc = 0.0f;
            for (int64_t b = 0; b < s.B; b++) {
                const int64_t ti = b * s.tiles_per_b + ct;
                const int64_t np = tile_pieces(s, ti);
                for (int64_t p = 0; p < np; p++)
                    acc += c.partA[((ti * s.pieces + p) * kWave + lane) * kH + j];
            }
            const float al = c.A_log[e];
            dA_log[e] = (al <= -10.0f || al >= 5.0f) ? 0.0f : acc * a_cont(al);
        } else {
            const int64_t d = i - nBC - nA;
            const int64_t ct = d / 32, q = d - ct * 32;
            float acc = 0.0f;
            for (int64_t b = 0; b < s.B; b++) {
                const int64_t ti = b * s.tiles_per_b + ct;
                const int64_t np = tile_pieces(s, ti);
                for (int64_t p = 0; p < np; p++) acc += c.partD[(ti * s.pieces + p) * 32 + q];
            }
            dD[d] = acc;
        }
    }
}

template <int DISC, int NS>
hipError_t launch_t(const BwdCols& c, const BwdShape& s, hipStream_t st) {
    hipLaunchKernelGGL((scan_bwd_kernel<DISC, NS>), dim3(static_cast<unsigned>(s.waves)),
                       dim3(kWave), 0, st, c, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs& a, const BwdShape& s, hipStream_t st) {
    BwdCols c{a.u,     a.delta, a.A_log, a.B,     a.C,     a.D_vec, a.z,
              a.h0,    a.h_ckpt, a.dout, a.du,    a.ddelta, a.dz,   a.dh0,
              a.ckpt,  a.partB, a.partC, a.partA, a.partD};
    hipError_t e;
    const bool vec = s.N == 16 && s.bc_vec;
    if (a.disc == MSS_DISC_EULER)
        e = vec ? launch_t<MSS_DISC_EULER, 16>(c, s, st) : launch_t<MSS_DISC_EULER, 0>(c, s, st);
    else
        e = vec ? launch_t<MSS_DISC_ZOH, 16>(c, s, st) : launch_t<MSS_DISC_ZOH, 0>(c, s, st);
    if (e != hipSuccess) return e;
    const int64_t total = s.B * s.L * (s.N == 16 ? 4 : s.N) + s.D * s.N + (a.dD_vec ? s.D : 0);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, c,
                       s, a.dB, a.dC, a.dA_log, a.dD_vec);
    return hipGetLastError();
}

}  // namespace mss
