// launch_ssd.h -- internal interface between the C-ABI layer (mss_api.hip)
// and the Mamba-2 SSD kernel.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mss.h"

namespace mss {

// One workgroup per (batch row, head, segment of seg_chunks chunks).
struct SsdArgs {
    int disc;              // MSS_DISC_ZOH or MSS_DISC_EULER
    int64_t B, L, H, P, N, G;
    int64_t nseg, seg_chunks;
    const float* x;        // (M, H*P)
    const float* dt;       // (M, H)
    const float* A_log;    // (H)
    const float* Bm;       // (M, G*N)
    const float* Cm;       // (M, G*N)
    const float* D_vec;    // (H) or null
    const float* dt_bias;  // (H) or null
    const float* h0;       // (B, H, P, N) or null
    float* y;              // (M, H*P)
    float* h_last;         // (B, H, P, N) or null
};

bool ssd_supported(int64_t P, int64_t N);
int ssd_chunk_len();
hipError_t launch_ssd(const SsdArgs& a, hipStream_t st);

}  // namespace mss
