// ssd_kernel.hip -- Mamba-2 state-space-dual (SSD) scan for gfx950 on the
// matrix cores.
//
// The recurrence the pages' Mamba2Block dispatches as ssd_chunk_forward
// (builderforce-memory-engine 2026.7.14 -> 2026.9.28, src/model/mamba2_block.ts:
// x (M, H*P), dt (M, H), B and C (M, G*N) split from the projections): per
// batch row and head h (group g = h / (H/G)), with A_h = -exp(clamp(A_log_h))
// and dv_t = softplus(dt_t + dt_bias_h),
//   S_t = exp(dv_t A_h) S_{t-1} + f_t x_t B_t^T      (S is P x N)
//   y_t = S_t C_t + D_h x_t
// where f_t = dv_t (EULER) or expm1(dv_t A_h) / A_h (ZOH), the two
// discretisations of the Mamba-1 path.
//
// Chunked form.  Over a chunk of Q steps with c_i = sum_{r<=i} dv_r A_h:
//   Y    = (L o C B^T) X  +  diag(e^{c}) C S_in^T...  (per head, P columns)
//   with L_ij = e^{c_i - c_j} f_j for i >= j (else 0), and
//   S_out = e^{c_{Q-1}} S_in + sum_j e^{c_{Q-1} - c_j} f_j x_j B_j^T.
// Every product is a dense contraction: v_mfma_f32_16x16x4f32 (fp32 in, fp32
// accumulate).  Indexing the summation as k = 4 (lane / 16) + step makes the
// accumulator layout of an S tile (rows n, columns p: lane l holds
// S[4 (l/16) + i][l % 16]) exactly the B operand of C S, so the state never
// leaves the registers between chunks.
//
// Mapping.  One workgroup (4 waves) per (batch row, head, time segment),
// three resident per CU for the common shapes (168 registers, under 53 KB of
// LDS).  Wave w owns the P columns [16 w c, ...) of S and of y.  Per chunk
// (its loads issued one chunk ahead into registers): X and B transposed, C,
// the decay prefix and the state weights go to LDS; the four waves share the
// work of the three nonzero 16 x 16 tiles of L o C B^T; each wave then forms
// its y columns and updates its S columns.  A segment that starts
// at t0 > 0 first rebuilds S(t0 - 1) by replaying the state update from the
// point where every contribution before it has decayed by 2^-c, with
// c = MSS_REPLAY_DECAY_BITS (for a scalar-decay head the walk is uniform
// across the head's channels), as the Mamba-1 kernels do.
#include "device_math.h"
#include "launch_ssd.h"

namespace mss {
namespace {

constexpr int kQ = 32;            // steps per chunk
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kCut = MSS_REPLAY_DECAY_BITS;   // replay until the carried part has decayed this many bits

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Global-memory pointers: accesses through them are global (not flat)
// instructions, which do not hold up the waits on LDS reads.
typedef const __attribute__((address_space(1))) float* gptr;
typedef const __attribute__((address_space(1))) v4f* gptr4;

// p + off as a scalar base the compiler cannot see through (so it is not
// split into one induction pointer per access).
__device__ __forceinline__ gptr gbase(const float* p, int64_t off) {
    gptr q = (gptr)(p) + off;
    asm volatile("" : "+s"(q));
    return q;
}

template <int P, int N>
struct Cfg {
    static constexpr int CT = P / 16;                   // column tiles of P
    static constexpr int CTW = CT >= kWaves ? CT / kWaves : 1;   // per wave
    static constexpr int NT = N / 16;
    static constexpr int LDN = N + 4;                   // C, B rows (floats)
    static constexpr int LDQ = kQ + 4;                  // Bt, Xt rows
    static constexpr int LDG = 16 + 4;                  // rows of a G tile
    static constexpr int GT = 16 * LDG;                 // one G tile (floats)
    // The three nonzero 16 x 16 tiles of L o C B^T (rows 0-15 x columns
    // 0-15, rows 16-31 x columns 0-15, rows 16-31 x columns 16-31) are
    // spread evenly over the four waves when the k tiles divide (BAL): each
    // tile is then the sum of two partial tiles, one in GA and one in GB.
    static constexpr bool BAL = NT % 4 == 0;
    // Waves per SIMD the registers are budgeted for: three workgroups per
    // CU (168 registers) where the state and the staged chunk fit in them.
    static constexpr int kWpe = P == 128 ? (N >= 128 ? 1 : N >= 64 ? 2 : 3) : 3;
    // LDS layout (floats)
    static constexpr int oC = 0;
    static constexpr int oBt = oC + kQ * LDN;
    static constexpr int oXt = oBt + N * LDQ;
    static constexpr int oGA = oXt + P * LDQ;
    static constexpr int oGB = oGA + 3 * GT;
    static constexpr int oCum = oGB + (BAL ? 3 * GT : 0);
    static constexpr int oDv = oCum + kQ;
    static constexpr int oW = oDv + kQ;
    static constexpr int oMisc = oW + kQ;
    static constexpr int total = oMisc + 4;
};

template <int P, int N>
struct Ssd {
    using C_ = Cfg<P, N>;
    const SsdArgs& a;
    const int64_t b, h, g;
    float* lds;
    const float A2;        // A_h log2(e)
    const float Ainv;      // 1 / A_h
    const float bias, dskip;
    const uint32_t lane, wave, q16, g4;   // lane, wave, lane % 16, lane / 16

    __device__ Ssd(const SsdArgs& a_, int64_t b_, int64_t h_, float* lds_)
        : a(a_), b(b_), h(h_), g(h_ / (a_.H / a_.G)), lds(lds_),
          A2(a_cont(a_.A_log[h_]) * kLog2e), Ainv(1.0f / a_cont(a_.A_log[h_])),
          bias(a_.dt_bias ? a_.dt_bias[h_] : 0.0f),
          dskip(a_.D_vec ? a_.D_vec[h_] : 0.0f), lane(threadIdx.x & 63u),
          wave(threadIdx.x >> 6), q16(threadIdx.x & 15u), g4((threadIdx.x & 63u) >> 4) {}

    __device__ __forceinline__ int64_t row(int64_t t) const { return b * a.L + t; }

    // The chunk's global data, held in registers between the load (issued
    // one chunk ahead) and the write to LDS.  Element idx of a tensor's chunk
    // is step j = idx % kQ and column (idx / kQ) * 4: consecutive lanes take
    // consecutive steps, so the transposed LDS writes (Xt, Bt) hit
    // consecutive banks.
    static constexpr int kXv = (kQ * (P / 4) + kThreads - 1) / kThreads;   // float4 per thread
    static constexpr int kBv = (kQ * (N / 4) + kThreads - 1) / kThreads;
    struct Stage {
        v4f xv[kXv], bv[kBv], cv[kBv];
        float dt;
    };

    // Loads of chunk [t0, t0 + kQ) (zeros past the sequence end, where dv = 0
    // leaves S unchanged and no output is written).  full: also C.  Each
    // tensor is read from the chunk's first row (a scalar base, made opaque
    // so that the compiler keeps one base instead of one pointer per load)
    // plus this lane's fixed offset; load k sits 32 floats past load k - 1.
    __device__ __forceinline__ void issue(Stage& st, int64_t t0, bool full) const {
        const int tid = threadIdx.x;
        const int64_t HP = a.H * P, GN = a.G * N;
        const int j = tid % kQ;
        const bool in = t0 + j < a.L;
        gptr xb = gbase(a.x, row(t0) * HP + h * P);
        gptr bb = gbase(a.Bm, row(t0) * GN + g * N);
        gptr cb = gbase(a.Cm, row(t0) * GN + g * N);
        const int64_t ox = j * HP + (tid / kQ) * 4, ob = j * GN + (tid / kQ) * 4;
        constexpr int kStep = (kThreads / kQ) * 4;
#pragma unroll
        for (int k = 0; k < kXv; k++) {
            v4f v = {0.f, 0.f, 0.f, 0.f};
            if (tid + k * kThreads < kQ * (P / 4) && in)
                v = *reinterpret_cast<gptr4>(xb + ox + k * kStep);
            st.xv[k] = v;
        }
#pragma unroll
        for (int k = 0; k < kBv; k++) {
            v4f vb = {0.f, 0.f, 0.f, 0.f}, vc = vb;
            if (tid + k * kThreads < kQ * (N / 4) && in) {
                vb = *reinterpret_cast<gptr4>(bb + ob + k * kStep);
                if (full)
                    vc = *reinterpret_cast<gptr4>(cb + ob + k * kStep);
            }
            st.bv[k] = vb;
            st.cv[k] = vc;
        }
        // wave 0 loads dt of its step (tid % kQ)
        float dtv = 0.0f;
        if (wave == 0 && in) dtv = a.dt[row(t0 + j) * a.H + h];
        st.dt = dtv;
    }

    // dv, the input factor f, the decay prefix c (log2 units) and the state
    // weight w_j = 2^{c_{Q-1} - c_j} f_j of step j = tid % kQ into LDS.  Run
    // by wave 0 alone (each 32-lane half; shuffles of width kQ): the other
    // waves go straight to the staging stores.
    __device__ __forceinline__ void decay_terms(const Stage& st, int64_t t0) const {
        const int tid = threadIdx.x;
        const int jj = tid % kQ;
        const float dv = t0 + jj < a.L ? softplus(st.dt + bias) : 0.0f;
        float cj = dv * A2;
        float fj = dv;
        if (a.disc == MSS_DISC_ZOH) {
            // expm1(dv A) / A; the cubic below |dv A| = 2^-6 keeps it exact
            // to ~2e-7 relative where aBar - 1 would cancel
            const float xn = cj * kLn2;
            const float p3 = xn * __builtin_fmaf(xn, __builtin_fmaf(xn, 1.0f / 6.0f, 0.5f), 1.0f);
            fj = (__builtin_fabsf(xn) < 0.015625f ? p3 : ex2(cj) - 1.0f) * Ainv;
        }
#pragma unroll
        for (int o = 1; o < kQ; o <<= 1) {
            const float v = __shfl_up(cj, o, kQ);
            if (jj >= o) cj += v;
        }
        const float last = __shfl(cj, kQ - 1, kQ);
        const float wj = ex2(last - cj) * fj;
        if (tid < kQ) {
            lds[C_::oCum + tid] = cj;
            lds[C_::oDv + tid] = fj;
            lds[C_::oW + tid] = wj;
        }
    }

    // Staged chunk into LDS: Xt and Bt (transposed), C, and f, the decay
    // prefix c (log2 units) and the state weights.  Ends with a barrier.
    __device__ __forceinline__ void commit(const Stage& st, int64_t t0) const {
        const int tid = threadIdx.x;
        if (wave == 0) decay_terms(st, t0);
        float* xt = lds + C_::oXt;
#pragma unroll
        for (int k = 0; k < kXv; k++) {
            const int i = tid + k * kThreads;
            if (i >= kQ * (P / 4)) break;
            const int j = i % kQ, p4 = (i / kQ) * 4;
            xt[(p4 + 0) * C_::LDQ + j] = st.xv[k].x;
            xt[(p4 + 1) * C_::LDQ + j] = st.xv[k].y;
            xt[(p4 + 2) * C_::LDQ + j] = st.xv[k].z;
            xt[(p4 + 3) * C_::LDQ + j] = st.xv[k].w;
        }
        float* bt = lds + C_::oBt;
#pragma unroll
        for (int k = 0; k < kBv; k++) {
            const int i = tid + k * kThreads;
            if (i >= kQ * (N / 4)) break;
            const int j = i % kQ, n4 = (i / kQ) * 4;
            *reinterpret_cast<v4f*>(lds + C_::oC + j * C_::LDN + n4) = st.cv[k];
            bt[(n4 + 0) * C_::LDQ + j] = st.bv[k].x;
            bt[(n4 + 1) * C_::LDQ + j] = st.bv[k].y;
            bt[(n4 + 2) * C_::LDQ + j] = st.bv[k].z;
            bt[(n4 + 3) * C_::LDQ + j] = st.bv[k].w;
        }
        __syncthreads();
    }

    // Partial G tile T (0: rows 0-15 x columns 0-15, 1: rows 16-31 x
    // columns 0-15, 2: rows 16-31 x columns 16-31) over the k tiles
    // [K0, K1) of N, scaled by 2^{c_i - c_j} f_j and masked to i >= j, into
    // tile T of dst.
    template <int T, int K0, int K1>
    __device__ __forceinline__ void g_part(float* dst) const {
        constexpr int ti = T == 0 ? 0 : 1, tj = T == 2 ? 1 : 0;
        // two accumulators over alternating halves of each k tile, added at
        // the end (independent chains for the matrix pipe)
        v4f acc = {0.f, 0.f, 0.f, 0.f}, acc2 = acc;
        const float* Cr = lds + C_::oC + (16 * ti + q16) * C_::LDN + 4 * g4;
        const float* Bc = lds + C_::oBt + 4 * g4 * C_::LDQ + 16 * tj + q16;
#pragma unroll
        for (int kt = K0; kt < K1; kt++) {
            const float4 ca = *reinterpret_cast<const float4*>(Cr + 16 * kt);
            const float* B0 = Bc + 16 * kt * C_::LDQ;
            acc = mfma(ca.x, B0[0], acc);
            acc2 = mfma(ca.y, B0[C_::LDQ], acc2);
            acc = mfma(ca.z, B0[2 * C_::LDQ], acc);
            acc2 = mfma(ca.w, B0[3 * C_::LDQ], acc2);
        }
        acc += acc2;
        const float* cum = lds + C_::oCum;
        const int j = 16 * tj + q16;
        const float cj = cum[j], dj = lds[C_::oDv + j];
        float* G = dst + T * C_::GT + q16;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int i = 16 * ti + 4 * g4 + r;
            G[(4 * g4 + r) * C_::LDG] = i >= j ? acc[r] * ex2(cum[i] - cj) * dj : 0.0f;
        }
    }

    // L o C B^T.  BAL: the 3 NT (tile, k tile) products in that order are
    // cut into four equal runs, one per wave; wave w's part of tile T goes
    // to GA when T = w, else to GB.  Otherwise waves 0-2 form one whole
    // tile each, into GA.
    __device__ __forceinline__ void form_g() const {
        constexpr int NT = C_::NT;
        float* GA = lds + C_::oGA;
        float* GB = lds + C_::oGB;
        if constexpr (C_::BAL) {
            constexpr int R = 3 * NT / 4;
            switch (wave) {
                case 0: g_part<0, 0, R>(GA); break;
                case 1: g_part<0, R, NT>(GB); g_part<1, 0, 2 * R - NT>(GA); break;
                case 2: g_part<1, 2 * R - NT, NT>(GB); g_part<2, 0, 3 * R - 2 * NT>(GA); break;
                default: g_part<2, 3 * R - 2 * NT, NT>(GB); break;
            }
        } else {
            switch (wave) {
                case 0: g_part<0, 0, NT>(GA); break;
                case 1: g_part<1, 0, NT>(GA); break;
                case 2: g_part<2, 0, NT>(GA); break;
                default: break;
            }
        }
    }

    // y for the chunk (rows < nout are written) = G X + diag(2^c) (C S) + D x.
    // The two 16-row tiles run interleaved (independent accumulation chains);
    // C S accumulates apart from G X so that its row scale 2^{c_i} is applied
    // once to the finished tile instead of to every operand.
    __device__ __forceinline__ void output(const v4f (&S)[C_::CTW][C_::NT], int64_t t0,
                                           int nout) const {
        const float* Xt = lds + C_::oXt;
        const float* Cc = lds + C_::oC;
        const float* cum = lds + C_::oCum;
        const int64_t HP = a.H * P;
        float f0[4], f1[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            f0[r] = ex2(cum[4 * g4 + r]);
            f1[r] = ex2(cum[16 + 4 * g4 + r]);
        }
        // this lane's A operands of the three G tiles (the same for every
        // column tile), partial tiles added
        float4 g00, g10, g11;
        {
            const float* ga = lds + C_::oGA + q16 * C_::LDG + 4 * g4;
            g00 = *reinterpret_cast<const float4*>(ga);
            g10 = *reinterpret_cast<const float4*>(ga + C_::GT);
            g11 = *reinterpret_cast<const float4*>(ga + 2 * C_::GT);
            if constexpr (C_::BAL) {
                const float* gb = ga + (C_::oGB - C_::oGA);
                const float4 b00 = *reinterpret_cast<const float4*>(gb);
                const float4 b10 = *reinterpret_cast<const float4*>(gb + C_::GT);
                const float4 b11 = *reinterpret_cast<const float4*>(gb + 2 * C_::GT);
                g00 = make_float4(g00.x + b00.x, g00.y + b00.y, g00.z + b00.z, g00.w + b00.w);
                g10 = make_float4(g10.x + b10.x, g10.y + b10.y, g10.z + b10.z, g10.w + b10.w);
                g11 = make_float4(g11.x + b11.x, g11.y + b11.y, g11.z + b11.z, g11.w + b11.w);
            }
        }
#pragma unroll
        for (int c = 0; c < C_::CTW; c++) {
            const int ct = wave * C_::CTW + c;
            if (ct >= C_::CT) break;
            v4f y0 = {0.f, 0.f, 0.f, 0.f}, y1 = y0, o0 = y0, o1 = y0;
            const float* Xr = Xt + (16 * ct + q16) * C_::LDQ + 4 * g4;
            // rows 0-15 see only the first 16 steps (the tile right of the
            // diagonal is zero and skipped)
            const float4 xb0 = *reinterpret_cast<const float4*>(Xr);
            const float4 xb1 = *reinterpret_cast<const float4*>(Xr + 16);
            y0 = mfma(g00.x, xb0.x, y0);
            y1 = mfma(g10.x, xb0.x, y1);
            y0 = mfma(g00.y, xb0.y, y0);
            y1 = mfma(g10.y, xb0.y, y1);
            y0 = mfma(g00.z, xb0.z, y0);
            y1 = mfma(g10.z, xb0.z, y1);
            y0 = mfma(g00.w, xb0.w, y0);
            y1 = mfma(g10.w, xb0.w, y1);
            y1 = mfma(g11.x, xb1.x, y1);
            y1 = mfma(g11.y, xb1.y, y1);
            y1 = mfma(g11.z, xb1.z, y1);
            y1 = mfma(g11.w, xb1.w, y1);
            const float* C0 = Cc + q16 * C_::LDN + 4 * g4;
            const float* C1 = C0 + 16 * C_::LDN;
#pragma unroll
            for (int tn = 0; tn < C_::NT; tn++) {
                const float4 c0 = *reinterpret_cast<const float4*>(C0 + 16 * tn);
                const float4 c1 = *reinterpret_cast<const float4*>(C1 + 16 * tn);
                o0 = mfma(c0.x, S[c][tn][0], o0);
                o1 = mfma(c1.x, S[c][tn][0], o1);
                o0 = mfma(c0.y, S[c][tn][1], o0);
                o1 = mfma(c1.y, S[c][tn][1], o1);
                o0 = mfma(c0.z, S[c][tn][2], o0);
                o1 = mfma(c1.z, S[c][tn][2], o1);
                o0 = mfma(c0.w, S[c][tn][3], o0);
                o1 = mfma(c1.w, S[c][tn][3], o1);
            }
            const int p = 16 * ct + q16;
            // x of rows 4 g4 .. 4 g4 + 3 (and 16 more) of column p: one
            // 16-byte read each
            const float4 x0 = *reinterpret_cast<const float4*>(Xt + p * C_::LDQ + 4 * g4);
            const float4 x1 = *reinterpret_cast<const float4*>(Xt + p * C_::LDQ + 16 + 4 * g4);
            const float xs0[4] = {x0.x, x0.y, x0.z, x0.w}, xs1[4] = {x1.x, x1.y, x1.z, x1.w};
            gptr yb = gbase(a.y, row(t0) * HP + h * P);
            auto* yr = const_cast<__attribute__((address_space(1))) float*>(yb) +
                       (static_cast<int64_t>(4 * g4) * HP + p);
            float v0[4], v1[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                v0[r] = __builtin_fmaf(dskip, xs0[r], __builtin_fmaf(f0[r], o0[r], y0[r]));
                v1[r] = __builtin_fmaf(dskip, xs1[r], __builtin_fmaf(f1[r], o1[r], y1[r]));
            }
            if (nout == kQ) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    yr[r * HP] = v0[r];
                    yr[(16 + r) * HP] = v1[r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    if (4 * g4 + r < nout) yr[r * HP] = v0[r];
                    if (16 + 4 * g4 + r < nout) yr[(16 + r) * HP] = v1[r];
                }
            }
        }
    }

    // S <- e^{c_{Q-1}} S + sum_j B_j^T (w_j x_j) (this wave's columns; the
    // weights go on the x operand in registers, so Bt stays unweighted for
    // the C B^T tiles).
    __device__ __forceinline__ void update(v4f (&S)[C_::CTW][C_::NT]) const {
        const float decay = ex2(lds[C_::oCum + kQ - 1]);
        const float* Bt = lds + C_::oBt;
        const float* Xt = lds + C_::oXt;
#pragma unroll
        for (int c = 0; c < C_::CTW; c++) {
            const int ct = wave * C_::CTW + c;
            if (ct >= C_::CT) break;
            const float* Xr = Xt + (16 * ct + q16) * C_::LDQ + 4 * g4;
            float4 xb[kQ / 16];
#pragma unroll
            for (int kt = 0; kt < kQ / 16; kt++) {
                const float4 wv = *reinterpret_cast<const float4*>(lds + C_::oW + 16 * kt + 4 * g4);
                const float4 xv = *reinterpret_cast<const float4*>(Xr + 16 * kt);
                xb[kt] = make_float4(xv.x * wv.x, xv.y * wv.y, xv.z * wv.z, xv.w * wv.w);
            }
#pragma unroll
            for (int tn = 0; tn < C_::NT; tn++) {
                v4f s = S[c][tn] * decay;
                const float* Br = Bt + (16 * tn + q16) * C_::LDQ + 4 * g4;
#pragma unroll
                for (int kt = 0; kt < kQ / 16; kt++) {
                    const float4 ba = *reinterpret_cast<const float4*>(Br + 16 * kt);
                    s = mfma(ba.x, xb[kt].x, s);
                    s = mfma(ba.y, xb[kt].y, s);
                    s = mfma(ba.z, xb[kt].z, s);
                    s = mfma(ba.w, xb[kt].w, s);
                }
                S[c][tn] = s;
            }
        }
    }

    // First step of the replay that rebuilds S(t0 - 1): walk dt backwards
    // until sum dv |A| >= c ln 2 (every contribution before it has decayed
    // by 2^-c), or t = 0.  One wave walks 64 steps at a time.
    __device__ __forceinline__ int64_t replay_start(int64_t t0) const {
        if (t0 == 0) return 0;
        int64_t* res = reinterpret_cast<int64_t*>(lds + C_::oMisc);
        if (wave == 0) {
            float total = 0.0f;
            int64_t t = t0;
            int64_t found = 0;
            while (t > 0) {
                const int64_t tt = t - 1 - static_cast<int64_t>(lane);   // lane 0 = newest
                const float dv = tt >= 0 ? softplus(a.dt[row(tt) * a.H + h] + bias) : 0.0f;
                float s = dv * -A2;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const float v = __shfl_up(s, o);
                    if (lane >= static_cast<uint32_t>(o)) s += v;
                }
                const uint64_t hit = __builtin_amdgcn_ballot_w64(tt >= 0 && total + s >= kCut);
                if (hit) {
                    found = t - 1 - static_cast<int64_t>(__builtin_ctzll(hit));
                    break;
                }
                total += __shfl(s, kWave - 1);
                t -= kWave;
            }
            if (lane == 0) *res = found > 0 ? found : 0;
        }
        __syncthreads();
        const int64_t r = *res;
        __syncthreads();
        return r;
    }
};

template <int P, int N>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Cfg<P, N>::kWpe)))
void ssd_kernel(SsdArgs a) {
    using C_ = Cfg<P, N>;
    __shared__ __align__(16) float lds[C_::total];
    const int64_t wg = blockIdx.x;
    const int64_t bh = wg / a.nseg;
    const int64_t sg = wg - bh * a.nseg;
    const int64_t b = bh / a.H, h = bh - b * a.H;
    const int64_t nchunks = (a.L + kQ - 1) / kQ;
    const int64_t c0 = sg * a.seg_chunks;
    const int64_t c1 = c0 + a.seg_chunks < nchunks ? c0 + a.seg_chunks : nchunks;
    Ssd<P, N> sd(a, b, h, lds);

    v4f S[C_::CTW][C_::NT];
    const int64_t tw = sd.replay_start(c0 * kQ);
    const int64_t cw = tw / kQ;
#pragma unroll
    for (int c = 0; c < C_::CTW; c++) {
        const int ct = sd.wave * C_::CTW + c;
#pragma unroll
        for (int tn = 0; tn < C_::NT; tn++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int n = 16 * tn + 4 * sd.g4 + r, p = 16 * ct + sd.q16;
                S[c][tn][r] = (cw == 0 && a.h0 && ct < C_::CT)
                                  ? a.h0[((b * a.H + h) * P + p) * N + n]
                                  : 0.0f;
            }
    }
    // Chunks [cw, c0) rebuild the state only; [c0, c1) also produce y.  The
    // loads of chunk c + 1 are in flight while chunk c computes.
    typename Ssd<P, N>::Stage st;
    sd.issue(st, cw * kQ, cw >= c0);
    for (int64_t c = cw; c < c1; c++) {
        const int64_t t0 = c * kQ;
        sd.commit(st, t0);
        if (c + 1 < c1) sd.issue(st, t0 + kQ, c + 1 >= c0);
        // The matrix-core phases run at raised wave priority, so that a
        // SIMD issues them ahead of another workgroup's staging work.
        __builtin_amdgcn_s_setprio(1);
        if (c >= c0) {
            sd.form_g();
            __syncthreads();
            const int nout = a.L - t0 < kQ ? static_cast<int>(a.L - t0) : kQ;
            sd.output(S, t0, nout);
        }
        sd.update(S);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
    }
    if (c1 == nchunks && a.h_last) {
#pragma unroll
        for (int c = 0; c < C_::CTW; c++) {
            const int ct = sd.wave * C_::CTW + c;
            if (ct >= C_::CT) break;
#pragma unroll
            for (int tn = 0; tn < C_::NT; tn++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int n = 16 * tn + 4 * sd.g4 + r, p = 16 * ct + sd.q16;
                    a.h_last[((b * a.H + h) * P + p) * N + n] = S[c][tn][r];
                }
        }
    }
}

template <int P, int N>
hipError_t launch_pn(const SsdArgs& a, hipStream_t st) {
    const int64_t nwg = a.B * a.H * a.nseg;
    hipLaunchKernelGGL((ssd_kernel<P, N>), dim3(static_cast<unsigned>(nwg)), dim3(kThreads), 0,
                       st, a);
    return hipGetLastError();
}

template <int P>
hipError_t launch_p(const SsdArgs& a, hipStream_t st) {
    switch (a.N) {
        case 16: return launch_pn<P, 16>(a, st);
        case 32: return launch_pn<P, 32>(a, st);
        case 64: return launch_pn<P, 64>(a, st);
        case 128: return launch_pn<P, 128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool ssd_supported(int64_t P, int64_t N) {
    return (P == 16 || P == 32 || P == 64 || P == 128) &&
           (N == 16 || N == 32 || N == 64 || N == 128);
}

int ssd_chunk_len() { return kQ; }

hipError_t launch_ssd(const SsdArgs& a, hipStream_t st) {
    switch (a.P) {
        case 16: return launch_p<16>(a, st);
        case 32: return launch_p<32>(a, st);
        case 64: return launch_p<64>(a, st);
        case 128: return launch_p<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mss
