// scan_kernel.hip -- selective scan (optionally fused with the causal conv1d +
// SiLU that produces its input) for gfx950.
//
// Computes mamba1CpuForward steps 4-5 (fused variant only), 8 and 9 of the
// Mamba-1 CPU mirror (builderforce-memory-engine 2026.7.12 -> 2026.9.27,
// src/training/mamba1_cpu.ts): per (b, d) column and time step t
//   u  = SiLU(bConv + sum_k wConv[d,k] x[t-k])      (fused variant; else u given)
//   dv = softplus(delta),  aBar_n = exp(dv * A_n)
//   h_n = aBar_n h_n + bBar_n u,   y = D u + sum_n C_n h_n,   out = y SiLU(z)
//
// Mapping.  One wave64 per work item; lane = channel d, so each lane owns the
// full N-state vector of its column in VGPRs and the N-reduction for y stays
// inside the lane.  Time advances in straight-line blocks of kT steps: at the
// start of a block the wave issues the loads of the next block (one 256-byte
// row segment per tensor and step, addressed as a uniform row base plus a
// 32-bit lane offset) and fetches the next block's B and C rows (1 KB, one
// 16-byte load per lane), which it stages through LDS; every step then reads
// its B_t / C_t with broadcast LDS loads, which cost no VALU issue slots.
// The path is VALU-bound (one v_exp_f32 per (t, d, n) at half the FMA rate
// plus ~4 FMA-class operations), so the per-step arithmetic is kept minimal.
//
// Parallelism over time.  The B * ceil(D/64) column tiles alone give too few
// waves for 1024 SIMDs, so the flattened (tile, t) space is cut into equal
// segments, one per wave.  A segment that starts at t0 > 0 needs the state
// h(t0 - 1) = sum_{s < t0} (prod_{r=s+1}^{t0-1} aBar_r) bBar_s u_s.  The
// recurrence forgets exponentially, so the wave sums these terms newest
// first, keeping each state's decay product q, and stops a state at the
// first 8-step block boundary where its q is below 2^-c in every lane
// (c = MSS_REPLAY_DECAY_BITS).  What that leaves out is q times the state
// before that step: small against the outputs unless that state is far
// larger than they are (~2^c / 10^4 times); reaching t = 0 (with h0) makes
// it exact.  MSS_FLAG_EXACT makes every segment a whole tile (no replay).
// No workspace and no inter-wave synchronisation.
#include "device_math.h"
#include "launch.h"

namespace mss {
namespace {

constexpr int kT = 8;                         // steps per straight-line block
// A state's replay stops once its decay to the segment start is below 2^-c.
constexpr float pow2_neg(int c) { return c <= 0 ? 1.0f : 0.5f * pow2_neg(c - 1); }
constexpr float kDropQ = pow2_neg(MSS_REPLAY_DECAY_BITS);
// Below |dv*A| = 2^-6 the decay is applied through expm1 (see step()).
constexpr float kSmallX = 0.015625f;
constexpr float kSmallX2 = kSmallX * kLog2e;  // the same bound in log2 units

struct Cols {
    const float* __restrict__ src;      // x (fused) or u, (M, D)
    const float* __restrict__ delta;    // (M, D)
    const float* __restrict__ A_log;    // (D, N)
    const float* __restrict__ Bm;       // (M, N)
    const float* __restrict__ Cm;       // (M, N)
    const float* __restrict__ Dv;       // (D) or null
    const float* __restrict__ z;        // (M, D) or null
    const float* __restrict__ h0;       // (B, D, N) or null
    const float* __restrict__ w_conv;   // (D, K) fused only
    const float* __restrict__ b_conv;   // (D) or null
    float* __restrict__ y;              // (M, D)
    float* __restrict__ h_cache;        // (B, L, D, N) or null
    float* __restrict__ h_last;         // (B, D, N) or null
};

// Per-lane constants and state of one (b, d) column.
template <int KS, int NS>
struct Lane {
    static constexpr int NR = NS > 0 ? NS : kMaxN;                   // register slots for states
    static constexpr int KR = KS > 0 ? KS : (KS == 0 ? kMaxK : 1);  // conv taps held
    float A2[NR];       // A * log2(e)
    float Ai[NR];       // 1 / A (ZOH only)
    float h[NR];
    float w[KR];
    float xw[KR > 1 ? KR - 1 : 1];  // xw[j] = conv input at t-1-j
    float bias, dvec, min_a2;
};

// Output modes of a sweep.
constexpr int kWarm = 0;     // state only
constexpr int kOut = 1;      // y
constexpr int kOutHC = 2;    // y and hCache
constexpr int kOutCK = 3;    // y and the state entering every 8th step

// State-cache modes of a kernel instantiation.
constexpr int kCacheNone = 0;
constexpr int kCacheAll = 1;     // h_cache (B, L, D, N): every step's state
constexpr int kCacheCk8 = 2;     // h_cache (B, ceil(L/8), D, N): the state entering steps 0, 8, 16, ...

// DN: every activation row stride is D and the B/C stride is N (dense
// tensors); the strides then fold into one row offset per step.
// CM: the state-cache mode (kCache*; each a kernel of its own, so that the
// staging of the state cache does not take registers from the kernel
// without it).
template <int DISC, int KS, int NS, bool DN, int CM>
struct Scan {
    using L_t = Lane<KS, NS>;
    static constexpr int NR = L_t::NR;
    static constexpr int KR = L_t::KR;
    static constexpr bool kFused = KS >= 0;
    static constexpr bool kStage = NS == 16;   // B/C rows staged through LDS
    // Alternating register sets for the block inputs where they fit without
    // spilling: dense rows, no state cache, a fixed conv width (the other
    // instantiations copy the prefetched set instead).
    static constexpr bool kPingPong = DN && CM == kCacheNone && KS != 0;

    const Cols& c;
    const int64_t L, D;
    const int N, K;
    const uint32_t d;       // this lane's channel, clamped to D-1
    const int64_t d0;       // the wave's first channel
    const int64_t b;
    const int64_t ldx, ldz, ldd, ldB, ldC, ldy;   // row strides (elements)
    const float* zsrc;      // z, or any valid array when ungated
    const bool gated;
    float4* lds;            // 64 float4 for this wave: B rows [0, 32), C rows [32, 64)
    float4* hst;            // N = 16 hCache staging: lane l's states at [5 l, 5 l + 4)

    // Lanes past D compute channel D-1 again and store bit-identical values to
    // the same addresses as lane D-1, so no store needs a lane mask.
    __device__ Scan(const Cols& c_, const ScanShape& s, int64_t b_, int64_t d_raw, float4* lds_,
                    float4* hst_)
        : c(c_), L(s.L), D(s.D), N(NS > 0 ? NS : s.N), K(KS > 0 ? KS : s.K),
          d(static_cast<uint32_t>(d_raw < s.D ? d_raw : s.D - 1)),
          d0(d_raw - static_cast<int64_t>(threadIdx.x)), b(b_),
          ldx(DN ? s.D : s.ld_src), ldz(DN ? s.D : (c_.z ? s.ld_z : s.ld_src)),
          ldd(DN ? s.D : s.ld_delta), ldB(DN ? N : s.ld_B), ldC(DN ? N : s.ld_C),
          ldy(DN ? s.D : s.ld_y),
          zsrc(c_.z ? c_.z : c_.src), gated(c_.z != nullptr), lds(lds_), hst(hst_) {}

    __device__ __forceinline__ int64_t row(int64_t t) const { return b * L + t; }
    __device__ __forceinline__ float ld(const float* base, int64_t stride, int64_t t) const {
        return (base + row(t) * stride)[d];
    }

    __device__ __forceinline__ void init(L_t& ln) const {
        float mn = 3.0e38f;
#pragma unroll
        for (int n = 0; n < NR; n++) {
            if (NS > 0 || n < N) {
                const float A = a_cont(c.A_log[d * N + n]);
                ln.A2[n] = A * kLog2e;
                ln.Ai[n] = 1.0f / A;
                mn = __builtin_fminf(mn, -ln.A2[n]);
            } else {            // padding state: never fed, never read
                ln.A2[n] = -1.0f;
                ln.Ai[n] = 0.0f;
            }
            ln.h[n] = 0.0f;
        }
        ln.min_a2 = mn;
        ln.dvec = c.Dv ? c.Dv[d] : 0.0f;
        if constexpr (kFused) {
            ln.bias = c.b_conv ? c.b_conv[d] : 0.0f;
#pragma unroll
            for (int k = 0; k < KR; k++) ln.w[k] = (KS > 0 || k < K) ? c.w_conv[d * K + k] : 0.0f;
        }
    }

    __device__ __forceinline__ void load_window(L_t& ln, int64_t t) const {
        if constexpr (kFused) {
#pragma unroll
            for (int j = 0; j < KR - 1; j++) {
                const int64_t tt = t - 1 - j;
                ln.xw[j] = (j < K - 1 && tt >= 0) ? ld(c.src, ldx, tt) : 0.0f;
            }
        }
    }

    // Inputs of steps t0 .. t0+kT-1; rows past the sequence end (the
    // prefetch after the last block starts at t0 = L) repeat its last row
    // and are never used.  Wave-uniform row pointers advance by one row
    // stride per step, so no step needs a row product.
    template <int OUT>
    __device__ __forceinline__ void load_block(float (&xs)[kT], float (&ds)[kT], float (&zs)[kT],
                                               int64_t t0) const {
        const int64_t s0 = t0 < L ? t0 : L - 1;
        const int64_t nv = L - s0;   // rows from s0 to the sequence end (>= 1)
        const float* px = c.src + row(s0) * ldx;
        const float* pd = c.delta + row(s0) * ldd;
        const float* pz = zsrc + row(s0) * ldz;
#pragma unroll
        for (int i = 0; i < kT; i++) {
            xs[i] = px[d];
            ds[i] = pd[d];
            if constexpr (OUT != kWarm) zs[i] = pz[d];
            if (i + 1 < nv) {
                px += ldx;
                pd += ldd;
                pz += ldz;
            }
        }
    }

    // This lane's 16 bytes of the B rows (lanes 0-31) or C rows (lanes 32-63)
    // of steps t0 .. t0+kT-1 (clamped to the last row like load_block).
    __device__ __forceinline__ float4 load_bc(int64_t t0) const {
        const uint32_t lane = threadIdx.x;
        const uint32_t q = lane & 31u;
        int64_t t = t0 + (q >> 2);
        t = t < L ? t : L - 1;
        const float* base = lane < 32 ? c.Bm + row(t) * ldB : c.Cm + row(t) * ldC;
        return *reinterpret_cast<const float4*>(base + (q & 3u) * 4);
    }

    // The scan input of one step: conv1d + SiLU of x (fused; advances the
    // conv window) or u itself.
    __device__ __forceinline__ float scan_input(L_t& ln, float xv) const {
        if constexpr (kFused) {
            float acc = __builtin_fmaf(ln.w[0], xv, ln.bias);
#pragma unroll
            for (int k = 1; k < KR; k++)
                if (KS > 0 || k < K) acc = __builtin_fmaf(ln.w[k], ln.xw[k - 1], acc);
#pragma unroll
            for (int j = KR - 2; j > 0; j--) ln.xw[j] = ln.xw[j - 1];
            if constexpr (KR > 1) ln.xw[0] = xv;
            return silu(acc);
        } else {
            return xv;
        }
    }

    // This wave's states, stored to the state-cache row `hc` ((D, N) of one
    // step).
    __device__ __forceinline__ void store_state(const L_t& ln, float* __restrict__ hc) const {
        if constexpr (NS == 16) {
            // The wave's 64 x 16 states of the step are one contiguous
            // 4 KB block: through LDS (80-byte lane stride, conflict
            // free) so that each 16-byte store instruction writes 1 KB
            // contiguously (a lane storing its own 64 bytes would
            // spread every store over 4 KB).  One wave per workgroup:
            // its LDS accesses complete in program order.
            const uint32_t lane = threadIdx.x;
#pragma unroll
            for (int j = 0; j < 4; j++)
                hst[5 * lane + j] = make_float4(ln.h[4 * j], ln.h[4 * j + 1],
                                                ln.h[4 * j + 2], ln.h[4 * j + 3]);
            float4* hb = reinterpret_cast<float4*>(hc + d0 * 16);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int q = i * kWave + static_cast<int>(lane);
                if (d0 + q / 4 < D) hb[q] = hst[5 * (q / 4) + (q % 4)];
            }
        } else if constexpr (NS > 0 && NS % 4 == 0) {
#pragma unroll
            for (int n = 0; n < NR; n += 4)
                *reinterpret_cast<float4*>(hc + d * NS + n) =
                    make_float4(ln.h[n], ln.h[n + 1], ln.h[n + 2], ln.h[n + 3]);
        } else {
#pragma unroll
            for (int n = 0; n < NR; n++)
                if (n < N) hc[d * N + n] = ln.h[n];
        }
    }

    // One time step.  SLOW: some lane has |dv A| < 2^-6 (see below).
    // LDS: B_t / C_t come from the staged block at row i; otherwise from
    // scalar loads.
    template <int OUT, bool SLOW, bool LDS>
    __device__ __forceinline__ void step(L_t& ln, float xv, float dv, float zv, int64_t t,
                                         int i) const {
        // The decays depend on dv alone: issued first, they overlap the
        // input's conv and SiLU and the B/C reads.
        float ab[NR];
        if constexpr (!SLOW) {
#pragma unroll
            for (int n = 0; n < NR; n++) ab[n] = ex2(dv * ln.A2[n]);
        }
        const float u = scan_input(ln, xv);
        float Bv[NR], Cv[NR];
        if constexpr (LDS) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 bq = lds[i * 4 + q];
                Bv[4 * q] = bq.x; Bv[4 * q + 1] = bq.y; Bv[4 * q + 2] = bq.z; Bv[4 * q + 3] = bq.w;
                if constexpr (OUT != kWarm) {
                    const float4 cq = lds[32 + i * 4 + q];
                    Cv[4 * q] = cq.x; Cv[4 * q + 1] = cq.y; Cv[4 * q + 2] = cq.z; Cv[4 * q + 3] = cq.w;
                }
            }
        } else {
            const cfloat* Br = as_const(c.Bm + row(t) * ldB);
            const cfloat* Cr = as_const(c.Cm + row(t) * ldC);
#pragma unroll
            for (int n = 0; n < NR; n++) {
                Bv[n] = (NS > 0 || n < N) ? Br[n] : 0.0f;
                if constexpr (OUT != kWarm) Cv[n] = (NS > 0 || n < N) ? Cr[n] : 0.0f;
            }
        }
        float yv = ln.dvec * u;
        if constexpr (!SLOW) {
            // |dv * A| >= 2^-6 in every lane and state: aBar <= 0.985, the
            // memory is short and aBar is used directly.
            if constexpr (DISC == MSS_DISC_EULER) {
                const float dvu = dv * u;
#pragma unroll
                for (int n = 0; n < NR; n++) {
                    if (NS > 0 || n < N) {
                        ln.h[n] = __builtin_fmaf(ab[n], ln.h[n], dvu * Bv[n]);
                        if constexpr (OUT != kWarm) yv = __builtin_fmaf(Cv[n], ln.h[n], yv);
                    }
                }
            } else {
                // h' = aBar (h + K) - K with K = u B / A  (= aBar h + (aBar - 1) K)
#pragma unroll
                for (int n = 0; n < NR; n++) {
                    if (NS > 0 || n < N) {
                        const float k = (u * ln.Ai[n]) * Bv[n];
                        ln.h[n] = __builtin_fmaf(ab[n], ln.h[n] + k, -k);
                        if constexpr (OUT != kWarm) yv = __builtin_fmaf(Cv[n], ln.h[n], yv);
                    }
                }
            }
        } else {
            // Some lane has a nearly-integrating state.  Carry the decay as
            // h + m h with m = aBar - 1 = expm1(dv A): fl(aBar) near 1 has an
            // absolute error of ~3e-8 that would compound over the long memory,
            // m has a relative one.  m is a cubic when |dv A| < 2^-6
            // (truncation < 2e-7 relative), else aBar - 1.
            const float dvu = dv * u;
#pragma unroll
            for (int n = 0; n < NR; n++) {
                if (NS > 0 || n < N) {
                    const float x2 = dv * ln.A2[n];
                    const float a = ex2(x2);
                    const float x = x2 * kLn2;
                    const float p = x * __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 6.0f, 0.5f), 1.0f);
                    const float m = __builtin_fabsf(x) < kSmallX ? p : a - 1.0f;
                    if constexpr (DISC == MSS_DISC_EULER) {
                        ln.h[n] = __builtin_fmaf(dvu, Bv[n], __builtin_fmaf(m, ln.h[n], ln.h[n]));
                    } else {
                        const float k = (u * ln.Ai[n]) * Bv[n];
                        ln.h[n] = __builtin_fmaf(m, ln.h[n] + k, ln.h[n]);
                    }
                    if constexpr (OUT != kWarm) yv = __builtin_fmaf(Cv[n], ln.h[n], yv);
                }
            }
        }
        if constexpr (OUT != kWarm) {
            const int64_t r = row(t);
            const float g = silu(zv);
            (c.y + r * ldy)[d] = gated ? yv * g : yv;
            if constexpr (OUT == kOutHC) {
                store_state(ln, c.h_cache + r * D * N);
            } else if constexpr (OUT == kOutCK) {
                // the state entering step t + 1, when that is a multiple of 8
                if (((t + 1) & 7) == 0 && t + 1 < L)
                    store_state(ln, c.h_cache + (b * ((L + 7) >> 3) + ((t + 1) >> 3)) * D * N);
            }
        }
    }

    // Steps t0 .. t0+cnt-1 one at a time (not unrolled): loads its own
    // inputs and makes the fast/slow choice per step.  Used for the slow
    // path, block remainders and B/C without LDS staging.
    // LDS: the block's B/C rows are staged (step i of the block at row i).
    template <int OUT, bool LDS>
    __device__ __forceinline__ void steps1(L_t& ln, int64_t t0, int cnt) const {
        for (int i = 0; i < cnt; i++) {
            const int64_t t = t0 + i;
            const float xv = ld(c.src, ldx, t);
            const float dv = softplus(ld(c.delta, ldd, t));
            const float zv = OUT != kWarm ? ld(zsrc, ldz, t) : 0.0f;
            if (!wave_any(dv * ln.min_a2 < kSmallX2))
                step<OUT, false, LDS>(ln, xv, dv, zv, t, i);
            else
                step<OUT, true, LDS>(ln, xv, dv, zv, t, i);
        }
    }

    // Steps [tb, te) of one sweep.  Full blocks of kT steps on the fast path
    // run as straight-line code on prefetched inputs; other blocks and the
    // remainder go through steps1.
    template <int OUT>
    __device__ __forceinline__ void sweep(L_t& ln, int64_t tb, int64_t te) const {
        if (tb >= te) return;
        if constexpr (!kStage) {
            for (int64_t t = tb; t < te; t += kT) {
                const int cnt = te - t < kT ? static_cast<int>(te - t) : kT;
                if constexpr (kStage) lds[threadIdx.x] = load_bc(t);
                steps1<OUT, kStage>(ln, t, cnt);
            }
        } else if constexpr (kPingPong) {
            // Two register sets take turns: a block runs on one while the
            // next block's inputs load into the other, with no copies between
            // blocks.
            float ax[kT], ad[kT], az[kT], bx[kT], bd[kT], bz[kT];
            float4 abc = load_bc(tb), bbc;
            load_block<OUT>(ax, ad, az, tb);
            int64_t t = tb;
            while (t + kT <= te) {
                block<OUT>(ln, t, ax, ad, az, abc, bx, bd, bz, bbc);
                t += kT;
                if (t + kT > te) {
                    if (t < te) {
                        lds[threadIdx.x] = bbc;
                        steps1<OUT, true>(ln, t, static_cast<int>(te - t));
                    }
                    return;
                }
                block<OUT>(ln, t, bx, bd, bz, bbc, ax, ad, az, abc);
                t += kT;
            }
            if (t < te) {
                lds[threadIdx.x] = abc;
                steps1<OUT, true>(ln, t, static_cast<int>(te - t));
            }
        } else {
            // one register set: the prefetched inputs are copied before the
            // next block's loads reuse it
            float nx[kT], nd[kT], nz[kT];
            float4 nbc = load_bc(tb);
            load_block<OUT>(nx, nd, nz, tb);
            int64_t t = tb;
            for (; t + kT <= te; t += kT) {
                float cx[kT], cz[kT], dv[kT];
                float sdv = 0.0f;
#pragma unroll
                for (int i = 0; i < kT; i++) {
                    cx[i] = nx[i];
                    cz[i] = nz[i];
                    dv[i] = softplus(nd[i]);
                    sdv += dv[i];
                }
                lds[threadIdx.x] = nbc;
                load_block<OUT>(nx, nd, nz, t + kT);
                nbc = load_bc(t + kT);
                run_block<OUT>(ln, t, cx, dv, cz, sdv);
            }
            if (t < te) {
                lds[threadIdx.x] = nbc;
                steps1<OUT, true>(ln, t, static_cast<int>(te - t));
            }
        }
    }

    // One full block [t, t + kT) on the inputs (xs, ds, zs, bc) loaded for
    // it, with the next block's loads issued into (nx, nd, nz, nbc).
    template <int OUT>
    __device__ __forceinline__ void block(L_t& ln, int64_t t, const float (&xs)[kT],
                                          const float (&ds)[kT], const float (&zs)[kT],
                                          const float4& bc, float (&nx)[kT], float (&nd)[kT],
                                          float (&nz)[kT], float4& nbc) const {
        float dv[kT];
        float sdv = 0.0f;
#pragma unroll
        for (int i = 0; i < kT; i++) {
            dv[i] = softplus(ds[i]);
            sdv += dv[i];
        }
        lds[threadIdx.x] = bc;
        load_block<OUT>(nx, nd, nz, t + kT);
        nbc = load_bc(t + kT);
        run_block<OUT>(ln, t, xs, dv, zs, sdv);
    }

    // The steps of a full block once its B/C rows are in LDS: straight-line
    // on the fast path when every lane's slowest state decays by at least
    // exp(-kT 2^-6) over the block (the rounding of aBar, absolute ~3e-8
    // next to 1, then compounds over at most ~64 steps of memory, and a
    // single step with tiny dv A adds one such error), else step by step.
    template <int OUT>
    __device__ __forceinline__ void run_block(L_t& ln, int64_t t, const float (&xs)[kT],
                                              const float (&dv)[kT], const float (&zs)[kT],
                                              float sdv) const {
        if (!wave_any(sdv * ln.min_a2 < kT * kSmallX2)) {
            // (checkpoints fall on block ends -- segments start at
            // multiples of 8 -- so the straight-line block has no
            // branch in it and the checkpoint follows it)
            constexpr int OB = OUT == kOutCK ? kOut : OUT;
#pragma unroll
            for (int i = 0; i < kT; i++) step<OB, false, true>(ln, xs[i], dv[i], zs[i], t + i, i);
            if constexpr (OUT == kOutCK)
                if (t + kT < L)
                    store_state(ln, c.h_cache + (b * ((L + 7) >> 3) + ((t + kT) >> 3)) * D * N);
        } else {
            steps1<OUT, true>(ln, t, kT);
        }
    }

    // ---- the state a segment starts from -------------------------------
    // h(t0-1) = sum_{s < t0} q_s bBar_s u_s + q_{-1} h0 with
    // q_s = prod_{r=s+1}^{t0-1} aBar_r, accumulated newest step first: q is
    // a running product per state, and state n stops at the first block
    // boundary where q_n < 2^-c in every lane -- what it leaves out is q_n
    // times the state before that step, at most 2^-c of it.  ZOH terms are
    // q (aBar - 1) u B / A: the running sum takes q (aBar - 1) u B and 1/A
    // multiplies it once at the end.  Blocks of kT steps are counted back
    // from t0, the loads of the next block in flight while one is summed
    // (two in flight pushed the kernel past 256 VGPRs into scratch);
    // reaching t = 0 adds the decayed h0 and is exact.

    // Inputs of the block [tb, tb + kT) (tb may be negative for the block
    // that reaches the sequence start): src at tb-(KR-1) .. tb+kT-1 (zero
    // before t = 0), delta at tb .. tb+kT-1, and (N = 16, staged) this
    // lane's 16 bytes of the block's B rows (lanes 0-31 hold them).
    struct RBlock {
        float xh[kT + KR - 1];
        float dd[kT];
        float4 bq;
    };

    __device__ __forceinline__ void rload(RBlock& r, int64_t tb) const {
#pragma unroll
        for (int j = 0; j < kT + KR - 1; j++) {
            const int64_t t = tb - (KR - 1) + j;
            const int64_t tc = t < 0 ? 0 : (t < L ? t : L - 1);
            const float v = ld(c.src, ldx, tc);
            r.xh[j] = t >= 0 ? v : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kT; i++) {
            const int64_t t = tb + i;
            r.dd[i] = ld(c.delta, ldd, t < 0 ? 0 : (t < L ? t : L - 1));
        }
        if constexpr (kStage) {
            const uint32_t q = threadIdx.x & 31u;
            int64_t t = tb + static_cast<int64_t>(q >> 2);
            t = t < 0 ? 0 : (t < L ? t : L - 1);
            r.bq = *reinterpret_cast<const float4*>(c.Bm + row(t) * ldB + (q & 3u) * 4);
        }
    }

    // One block of the replay, newest step first.  FULL: no step before t = 0.
    // LAST: the block that reaches t = 0 (no state stops after it).
    template <bool FULL>
    __device__ __forceinline__ void rblock(const L_t& ln, const RBlock& r, int64_t tb,
                                           float (&q)[NR], float (&g)[NR], uint32_t& act,
                                           bool last) const {
        float dv[kT], w[kT];   // w: EULER dv u, ZOH u
        float sdv = 0.0f;
        int nst = 0;
#pragma unroll
        for (int i = 0; i < kT; i++) {
            if (FULL || tb + i >= 0) {
                dv[i] = softplus(r.dd[i]);
                float u;
                if constexpr (kFused) {
                    float acc = __builtin_fmaf(ln.w[0], r.xh[i + KR - 1], ln.bias);
#pragma unroll
                    for (int k = 1; k < KR; k++)
                        if (KS > 0 || k < K) acc = __builtin_fmaf(ln.w[k], r.xh[i + KR - 1 - k], acc);
                    u = silu(acc);
                } else {
                    u = r.xh[i];
                }
                w[i] = DISC == MSS_DISC_EULER ? dv[i] * u : u;
                sdv += dv[i];
                nst++;
            } else {
                dv[i] = 0.0f;
                w[i] = 0.0f;
            }
        }
        // The accurate form when the block's decay is weak in some lane, as
        // in the sweep: q (aBar - 1) from m = expm1(dv A) instead of q aBar - q.
        const bool slow = wave_any(sdv * ln.min_a2 < static_cast<float>(nst) * kSmallX2);
        if (!slow)
            rstates<FULL, false>(ln, tb, dv, w, q, g, act, last);
        else
            rstates<FULL, true>(ln, tb, dv, w, q, g, act, last);
    }

    // The states of one replay block (the block's inputs already reduced to
    // dv and w); ACC: the accurate form.
    template <bool FULL, bool ACC>
    __device__ __forceinline__ void rstates(const L_t& ln, int64_t tb, const float (&dv)[kT],
                                            const float (&w)[kT], float (&q)[NR], float (&g)[NR],
                                            uint32_t& act, bool last) const {
        const float* ldsf = reinterpret_cast<const float*>(lds);
#pragma unroll
        for (int n = 0; n < NR; n++) {
            if (!(act & (1u << n))) continue;
            float qq = q[n], gg = g[n];
#pragma unroll
            for (int i = kT - 1; i >= 0; i--) {
                if (!FULL && tb + i < 0) continue;
                float Bv;
                if constexpr (kStage) {
                    Bv = ldsf[i * 16 + n];
                } else {
                    Bv = as_const(c.Bm + row(tb + i) * ldB)[n];
                }
                const float x2 = dv[i] * ln.A2[n];
                const float a = ex2(x2);
                if constexpr (!ACC) {
                    if constexpr (DISC == MSS_DISC_EULER) {
                        gg = __builtin_fmaf(qq, w[i] * Bv, gg);
                        qq *= a;
                    } else {
                        const float qn = qq * a;
                        gg = __builtin_fmaf(qn - qq, w[i] * Bv, gg);
                        qq = qn;
                    }
                } else {
                    const float x = x2 * kLn2;
                    const float p = x * __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 6.0f, 0.5f), 1.0f);
                    const float m = __builtin_fabsf(x) < kSmallX ? p : a - 1.0f;
                    const float dq = qq * m;
                    if constexpr (DISC == MSS_DISC_EULER)
                        gg = __builtin_fmaf(qq, w[i] * Bv, gg);
                    else
                        gg = __builtin_fmaf(dq, w[i] * Bv, gg);
                    qq += dq;
                }
            }
            q[n] = qq;
            g[n] = gg;
            // Stop the state once its decay to t0 is below the cut in every
            // lane (a NaN never compares below: such a column runs to t = 0).
            if (!last && wave_all(qq < kDropQ)) act &= ~(1u << n);
        }
    }

    __device__ __forceinline__ void rebuild(L_t& ln, int64_t t0) const {
        float q[NR], g[NR];
        uint32_t act = 0;
#pragma unroll
        for (int n = 0; n < NR; n++) {
            q[n] = 1.0f;
            g[n] = 0.0f;
            if (NS > 0 || n < N) act |= 1u << n;
        }
        RBlock nxt;
        int64_t tb = t0 - kT;
        rload(nxt, tb);
        while (true) {
            // the block at tb; the loads of the one before it go out first
            if constexpr (kStage)
                if (threadIdx.x < 32) lds[threadIdx.x] = nxt.bq;
            const RBlock cur = nxt;
            if (tb > 0) rload(nxt, tb - kT);
            if (tb >= 0)
                rblock<true>(ln, cur, tb, q, g, act, tb == 0);
            else
                rblock<false>(ln, cur, tb, q, g, act, true);
            if (tb <= 0 || !act) break;
            tb -= kT;
        }
        // states still running here took every step down to t = 0
        const bool start = tb <= 0;
#pragma unroll
        for (int n = 0; n < NR; n++) {
            if (!(NS > 0 || n < N)) continue;
            float h = DISC == MSS_DISC_EULER ? g[n] : g[n] * ln.Ai[n];
            if (start && c.h0 && (act & (1u << n)))
                h = __builtin_fmaf(q[n], c.h0[(b * D + d) * N + n], h);
            ln.h[n] = h;
        }
    }

    // Produce outputs for steps [t0, t1) of this column.
    __device__ __forceinline__ void run(int64_t t0, int64_t t1) const {
        L_t ln;
        init(ln);
        if (t0 > 0) {
            rebuild(ln, t0);
        } else if (c.h0) {
#pragma unroll
            for (int n = 0; n < NR; n++)
                if (NS > 0 || n < N) ln.h[n] = c.h0[(b * D + d) * N + n];
        }
        load_window(ln, t0);
        if constexpr (CM == kCacheAll) {
            sweep<kOutHC>(ln, t0, t1);
        } else if constexpr (CM == kCacheCk8) {
            if (t0 == 0) store_state(ln, c.h_cache + b * ((L + 7) >> 3) * D * N);
            sweep<kOutCK>(ln, t0, t1);
        } else {
            sweep<kOut>(ln, t0, t1);
        }
        if (t1 == L && c.h_last) {
#pragma unroll
            for (int n = 0; n < NR; n++)
                if (NS > 0 || n < N) c.h_last[(b * D + d) * N + n] = ln.h[n];
        }
    }
};

// Two waves per SIMD: one wave alone issues VALU work only about every other
// slot, so the register budget is capped at 256 VGPRs.
template <int DISC, int KS, int NS, bool DN, int CM>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void scan_kernel(
    Cols c, ScanShape s) {
    __shared__ float4 lds[kWave];
    __shared__ float4 hst[NS == 16 && CM != kCacheNone ? 5 * kWave : 1];
    const int64_t lane = threadIdx.x;
    const int64_t g0 = static_cast<int64_t>(blockIdx.x) * s.seg;
    const int64_t g1 = g0 + s.seg < s.total ? g0 + s.seg : s.total;
    // A segment of the flattened (tile, t) space may cover the end of one
    // tile and the start of the next; walk its pieces.  Tiles are padded to
    // Lp steps (a multiple of 8) and segments are multiples of 8 long, so
    // every piece starts at a multiple of 8; the padding is skipped.
    for (int64_t g = g0; g < g1;) {
        const int64_t tile = g / s.Lp;
        const int64_t t0 = g - tile * s.Lp;
        if (t0 >= s.L) {
            g = (tile + 1) * s.Lp;
            continue;
        }
        const int64_t t1 = t0 + (g1 - g) < s.L ? t0 + (g1 - g) : s.L;
        const int64_t b = tile / s.tiles_per_b;
        const int64_t dt = tile - b * s.tiles_per_b;
        Scan<DISC, KS, NS, DN, CM> sc(c, s, b, dt * kWave + lane, lds, hst);
        sc.run(t0, t1);
        g += t1 - t0;
    }
}

template <int DISC, int KS, int NS, bool DN>
hipError_t launch_t(const Cols& c, const ScanShape& s, hipStream_t st) {
    const int64_t nblk = (s.total + s.seg - 1) / s.seg;
    const dim3 grid(static_cast<unsigned>(nblk));
    if (c.h_cache && s.ckpt8)
        hipLaunchKernelGGL((scan_kernel<DISC, KS, NS, DN, kCacheCk8>), grid, dim3(kWave), 0, st, c,
                           s);
    else if (c.h_cache)
        hipLaunchKernelGGL((scan_kernel<DISC, KS, NS, DN, kCacheAll>), grid, dim3(kWave), 0, st, c,
                           s);
    else
        hipLaunchKernelGGL((scan_kernel<DISC, KS, NS, DN, kCacheNone>), grid, dim3(kWave), 0, st,
                           c, s);
    return hipGetLastError();
}

template <int DISC, int KS>
hipError_t launch_n(const Cols& c, const ScanShape& s, hipStream_t st) {
    if (s.N == 16 && s.bc_vec)
        return s.dense ? launch_t<DISC, KS, 16, true>(c, s, st)
                       : launch_t<DISC, KS, 16, false>(c, s, st);
    return launch_t<DISC, KS, 0, false>(c, s, st);
}

template <int DISC>
hipError_t launch_k(const Cols& c, const ScanShape& s, hipStream_t st, bool fused) {
    if (!fused) return launch_n<DISC, -1>(c, s, st);
    return s.K == 4 ? launch_n<DISC, 4>(c, s, st) : launch_n<DISC, 0>(c, s, st);
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, const ScanShape& s, hipStream_t st) {
    Cols c{a.src, a.delta, a.A_log, a.B, a.C, a.D_vec, a.z, a.h0, a.w_conv, a.b_conv,
           a.y, a.h_cache, a.h_last};
    return a.disc == MSS_DISC_EULER ? launch_k<MSS_DISC_EULER>(c, s, st, a.fused)
                                    : launch_k<MSS_DISC_ZOH>(c, s, st, a.fused);
}

}  // namespace mss
