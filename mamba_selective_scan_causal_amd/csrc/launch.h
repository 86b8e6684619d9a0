// launch.h -- internal interface between the C-ABI layer (mss_api.hip) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mss.h"

namespace mss {

// Work split of a scan launch: the flattened (column tile, t) space of
// `total = B * tiles_per_b * Lp` steps (each tile padded to Lp = L rounded up
// to a multiple of 8) is cut into segments of `seg` steps (a multiple of 8),
// one wave64 each.
struct ScanShape {
    int64_t B, L, Lp, D;
    int N, K;
    int64_t tiles_per_b;
    int64_t total;
    int64_t seg;
    // row strides in elements (D, D, D, N, N, D when dense)
    int64_t ld_src, ld_z, ld_delta, ld_B, ld_C, ld_y;
    bool bc_vec;              // B and C rows 16-byte aligned: staged block loads
    bool dense;               // strides are exactly D (activations) and N (B, C)
    bool ckpt8;               // h_cache holds the state entering every 8th step
};

struct ScanArgs {
    int disc;
    bool fused;               // src is x (conv1d + SiLU fused) rather than u
    const float* src;
    const float* delta;
    const float* A_log;
    const float* B;
    const float* C;
    const float* D_vec;
    const float* z;
    const float* h0;
    const float* w_conv;
    const float* b_conv;
    float* y;
    float* h_cache;
    float* h_last;
};

hipError_t launch_scan(const ScanArgs& a, const ScanShape& s, hipStream_t st);

struct ConvArgs {
    int64_t B, L, D;
    int K;
    const float* x;
    const float* w_conv;
    const float* b_conv;
    float* u;
};

hipError_t launch_conv1d_silu(const ConvArgs& a, hipStream_t st);

struct StepArgs {
    int disc;
    int64_t B, D;
    int N, K;
    const float* x;
    const float* z;
    const float* delta;
    const float* A_log;
    const float* B_in;
    const float* C_in;
    const float* D_vec;
    const float* w_conv;
    const float* b_conv;
    float* conv_state;
    float* h;
    float* y;
};

hipError_t launch_step(const StepArgs& a, hipStream_t st);

// h_last for a zero-length sequence: h0 copied, or zeros.
hipError_t launch_state_init(const float* h0, float* h_last, int64_t count, hipStream_t st);

}  // namespace mss
