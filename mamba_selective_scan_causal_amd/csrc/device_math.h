// device_math.h -- fp32 elementwise functions of the Mamba-1 block core for
// gfx950, built on the hardware transcendental instructions.
//
// Measured on MI355X: v_exp_f32 <= 0.78 ulp, v_log_f32 <= 1 ulp (relative,
// including arguments next to 1), v_rcp_f32 <= 0.88 ulp; each issues at half
// the fp32 FMA rate and does not overlap FMAs, so every call here counts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mss {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kWave = 64;
constexpr int kMaxN = 16;
constexpr int kMaxK = 8;

__device__ __forceinline__ float ex2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float lg2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// SiLU(v) = v / (1 + e^-v)  (cpu_ops.ts, silu).  For v -> -inf the
// exponential overflows to +inf and the reciprocal gives 0, the right limit.
__device__ __forceinline__ float silu(float v) { return v * rcp(1.0f + ex2(-kLog2e * v)); }

// softplus(v) = max(v, 0) + log1p(e^-|v|)  (cpu_ops.ts, softplus).
// log1p(e) for e in (0, 1] is log(w) + (1 + e - w)/w with w = fl(1 + e); the
// rounding error c = e - (w - 1) is exact in fp32 (Sterbenz), and replacing
// c/w by c changes the result by at most c*e/(1+e), i.e. below 6e-8 relative.
// When e < 2^-24, w == 1 and the result is exactly e, so very negative inputs
// keep full relative accuracy.
__device__ __forceinline__ float softplus(float v) {
    const float e = ex2(-kLog2e * __builtin_fabsf(v));
    const float w = 1.0f + e;
    const float c = e - (w - 1.0f);
    return __builtin_fmaxf(v, 0.0f) + __builtin_fmaf(lg2(w), kLn2, c);
}

// Continuous A = -exp(clamp(A_log, -10, 5))  (mamba1CpuForward step 8,
// A_LOG_CLAMP_LO/HI).  Evaluated once per (d, n) with the accurate libm exp.
__device__ __forceinline__ float a_cont(float a_log) {
    const float c = __builtin_fminf(__builtin_fmaxf(a_log, -10.0f), 5.0f);
    return -expf(c);
}

// Read-only, wave-uniform rows (B_t, C_t) are read through the constant
// address space so that they become scalar loads into SGPRs, which VALU
// instructions take as operands at no cost.
typedef const __attribute__((address_space(4))) float cfloat;
__device__ __forceinline__ const cfloat* as_const(const float* p) { return (const cfloat*)p; }

// The same A from the hardware exponential (relative error ~|c| 6e-8 + 1 ulp,
// at most ~4e-7), for kernels that rebuild A on every call.
__device__ __forceinline__ float a_cont_fast(float a_log) {
    const float c = __builtin_fminf(__builtin_fmaxf(a_log, -10.0f), 5.0f);
    return -ex2(c * kLog2e);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
__device__ __forceinline__ bool wave_all(bool p) { return __builtin_amdgcn_ballot_w64(!p) == 0; }

}  // namespace mss
