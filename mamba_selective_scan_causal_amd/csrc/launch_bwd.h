// launch_bwd.h -- internal interface between the C-ABI layer (mss_api.hip)
// and the backward kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mss.h"

namespace mss {

// Backward of the scan: the flattened (tile, t) space of the B * tiles_per_b
// channel tiles (batch row, 32 channels), each tile padded to Lp = L rounded
// up to a multiple of 8 steps, is cut into `waves` segments of `seg` steps
// (a multiple of 8), one wave each; so every piece starts at a multiple of
// 8.  A segment crossing the end of a tile is worked as one piece per tile
// (the padding steps are skipped), and a tile has at most `pieces` pieces.
// Workspace regions (all fp32):
//   ckpt  (waves, blocks_per_seg, 64, 8)   h at every 8-step block start
//                                          (absent when the forward's checkpoints are given)
//   partB, partC (B, tiles_per_b, L, 16)    per-tile dB / dC rows
//   partA (tiles, pieces, 64, 8), partD (tiles, pieces, 32)  per-piece dA / dD sums
struct BwdShape {
    int64_t B, L, Lp, D;
    int N;
    int64_t tiles_per_b;      // ceil(D / 32)
    int64_t total;            // B * tiles_per_b * Lp
    int64_t seg, waves, blocks_per_seg, pieces;
    bool bc_vec;              // B and C rows 16-byte aligned (N = 16)
};

struct BwdArgs {
    int disc;
    const float* u;
    const float* delta;
    const float* A_log;
    const float* B;
    const float* C;
    const float* D_vec;
    const float* z;
    const float* h0;
    const float* h_ckpt;      // (B, ceil(L/8), D, N): the forward's state entering steps 0, 8, ... or null
    const float* dout;
    float* du;
    float* ddelta;
    float* dA_log;
    float* dB;
    float* dC;
    float* dD_vec;
    float* dz;
    float* dh0;
    float* ckpt;
    float* partB;
    float* partC;
    float* partA;
    float* partD;
};

hipError_t launch_scan_bwd(const BwdArgs& a, const BwdShape& s, hipStream_t st);

// Backward of conv1d + SiLU: one wave per (64-channel tile, group); group g
// takes the (b, 32-step run) jobs g, g + groups, ...  Workspace: part
// (tiles, groups, kMaxK + 1, 64) fp32, per-wave sums of dw (rows 0..K-1)
// and db (row K).
struct ConvBwdArgs {
    int64_t B, L, D;
    int K;
    int64_t groups;
    const float* x;
    const float* w_conv;
    const float* b_conv;
    const float* du;
    float* dx;
    float* dw;
    float* db;
    float* part;
};

hipError_t launch_conv1d_silu_bwd(const ConvBwdArgs& a, hipStream_t st);

}  // namespace mss
