// abi_sanitized.cpp -- host-side argument validation of libmss under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built by tests/test_abi_sanitized.py against a copy of the library whose
// host code (the extern "C" entry points of mss_api.hip) carries the
// sanitizers.  Every call below is rejected by validation before any HIP
// call, so the program needs no GPU; the pointers are never dereferenced.
// The size arithmetic is driven to its limits (int64 products that
// overflow, strides, empty problems with huge widths) so that a signed
// overflow or an out-of-bounds host access in the checks is reported.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "mss.h"

namespace {

int g_failed = 0;

void expect(int got, int want, const char* what) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
        g_failed++;
    }
}

// Distinct, 256-byte aligned, never dereferenced addresses, 16 MiB apart.
float* fake(int i) {
    return reinterpret_cast<float*>(static_cast<uintptr_t>(0x7f0000000000ull) +
                                    static_cast<uintptr_t>(i) * (16ull << 20));
}
float* misaligned(int i) { return reinterpret_cast<float*>(reinterpret_cast<char*>(fake(i)) + 8); }

mss_dims dims(int64_t b, int64_t l, int64_t d, int64_t n, int64_t k) {
    mss_dims x;
    x.struct_size = sizeof(mss_dims);
    x.flags = 0;
    x.batch = b;
    x.seq_len = l;
    x.d_inner = d;
    x.d_state = n;
    x.d_conv = k;
    return x;
}

mss_ssd_dims ssd_dims(int64_t b, int64_t l, int64_t h, int64_t p, int64_t n, int64_t g) {
    mss_ssd_dims x;
    x.struct_size = sizeof(mss_ssd_dims);
    x.flags = 0;
    x.batch = b;
    x.seq_len = l;
    x.n_heads = h;
    x.head_dim = p;
    x.d_state = n;
    x.n_groups = g;
    return x;
}

int scan(const mss_dims* d, int disc, float* u, float* y) {
    return mss_selective_scan(d, disc, u, fake(2), fake(3), fake(4), fake(5), nullptr, nullptr,
                              nullptr, y, nullptr, nullptr, nullptr);
}

int core(const mss_dims* d, float* x, float* w, float* y) {
    return mss_mamba1_core(d, MSS_DISC_ZOH, x, w, nullptr, fake(2), fake(3), fake(4), fake(5),
                           nullptr, nullptr, nullptr, y, nullptr, nullptr, nullptr);
}

int step(const mss_dims* d, float* x, float* h) {
    return mss_selective_step(d, MSS_DISC_EULER, x, nullptr, fake(2), fake(3), fake(4), fake(5),
                              nullptr, fake(6), nullptr, fake(7), h, fake(8), nullptr);
}

int scan_bwd(const mss_dims* d, float* du, void* ws, size_t ws_bytes) {
    return mss_selective_scan_backward(d, MSS_DISC_ZOH, fake(1), fake(2), fake(3), fake(4),
                                       fake(5), nullptr, nullptr, nullptr, nullptr, fake(6), du,
                                       fake(8), fake(9), fake(10), fake(11), nullptr, nullptr,
                                       nullptr, ws, ws_bytes, nullptr);
}

int conv_bwd(const mss_dims* d, float* dx, void* ws, size_t ws_bytes) {
    return mss_conv1d_silu_backward(d, fake(1), fake(2), nullptr, fake(3), dx, fake(5), nullptr,
                                    ws, ws_bytes, nullptr);
}

int ssd(const mss_ssd_dims* d, float* x, float* y) {
    return mss_ssd_scan(d, MSS_DISC_EULER, x, fake(2), fake(3), fake(4), fake(5), nullptr,
                        nullptr, nullptr, y, nullptr, nullptr);
}

}  // namespace

int main() {
    const int64_t big = int64_t(1) << 62;
    expect(mss_version(), MSS_VERSION, "version");
    for (int s = -6; s <= 1; s++)
        if (!mss_strerror(s)) expect(1, 0, "strerror");

    // sizes and the struct guard
    mss_dims d = dims(2, 64, 128, 16, 4);
    expect(scan(nullptr, 0, fake(1), fake(9)), MSS_EINVAL, "scan: null dims");
    mss_dims bad = d;
    bad.struct_size = 8;
    expect(scan(&bad, 0, fake(1), fake(9)), MSS_EINVAL, "scan: struct_size");
    bad = d;
    bad.flags = 4;
    expect(scan(&bad, 0, fake(1), fake(9)), MSS_EINVAL, "scan: unknown flag");
    mss_dims n17 = dims(2, 64, 128, 17, 4);
    expect(scan(&n17, 0, fake(1), fake(9)), MSS_EINVAL, "scan: N = 17");
    expect(scan(&d, 7, fake(1), fake(9)), MSS_EINVAL, "scan: disc");
    mss_dims neg = dims(-1, 64, 128, 16, 4);
    expect(scan(&neg, 0, fake(1), fake(9)), MSS_EINVAL, "scan: negative batch");
    mss_dims huge = dims(big, big, big, 16, 4);
    expect(scan(&huge, 0, fake(1), fake(9)), MSS_EINVAL, "scan: overflowing M D");
    mss_dims huge2 = dims(1, big / 4, 8, 16, 4);
    expect(scan(&huge2, 0, fake(1), fake(9)), MSS_EINVAL, "scan: overflowing bytes");
    expect(scan(&d, 0, misaligned(1), fake(9)), MSS_EALIGN, "scan: alignment");
    expect(scan(&d, 0, fake(1), fake(1)), MSS_EALIAS, "scan: y aliases u");
    expect(scan(&d, 0, nullptr, fake(9)), MSS_EINVAL, "scan: u missing");

    // fused core: conv weights, K limits, an empty sequence with a huge width
    expect(core(&d, fake(1), nullptr, fake(9)), MSS_EINVAL, "core: w_conv missing");
    mss_dims k9 = dims(2, 64, 128, 16, 9);
    expect(core(&k9, fake(1), fake(6), fake(9)), MSS_EINVAL, "core: K = 9");
    mss_dims wide = dims(1, 0, big, 1, 4);
    expect(core(&wide, fake(1), fake(6), fake(9)), MSS_EINVAL, "core: D K overflow, L = 0");
    expect(mss_conv1d_silu(&wide, fake(1), fake(6), nullptr, fake(9), nullptr), MSS_EINVAL,
           "conv: D K overflow, L = 0");
    expect(mss_conv1d_silu(&d, fake(1), fake(6), nullptr, fake(1), nullptr), MSS_EALIAS,
           "conv: u aliases x");

    // strided: a stride below the row width, and a span that overflows
    mss_strides st;
    st.struct_size = sizeof(mss_strides);
    st.reserved = 0;
    st.x = st.z = st.delta = st.y = 128;
    st.B = st.C = 16;
    mss_strides narrow = st;
    narrow.delta = 64;
    expect(mss_selective_scan_strided(&d, &narrow, 0, fake(1), fake(2), fake(3), fake(4), fake(5),
                                      nullptr, nullptr, nullptr, fake(9), nullptr, nullptr,
                                      nullptr),
           MSS_EINVAL, "strided: stride < width");
    mss_strides far = st;
    far.x = big;
    expect(mss_mamba1_core_strided(&d, &far, 0, fake(1), fake(6), nullptr, fake(2), fake(3),
                                   fake(4), fake(5), nullptr, nullptr, nullptr, fake(9), nullptr,
                                   nullptr, nullptr),
           MSS_EINVAL, "strided: span overflow");
    expect(mss_selective_scan_strided(&d, nullptr, 0, fake(1), fake(2), fake(3), fake(4), fake(5),
                                      nullptr, nullptr, nullptr, fake(9), nullptr, nullptr,
                                      nullptr),
           MSS_EINVAL, "strided: null strides");

    // decode step
    mss_dims sd = dims(4, 1, 128, 16, 4);
    expect(step(&sd, fake(1), fake(1)), MSS_EALIAS, "step: h aliases x");
    mss_dims swide = dims(0, 1, big, 1, 4);
    expect(step(&swide, fake(1), fake(9)), MSS_EINVAL, "step: D K overflow, B = 0");

    // backward: workspace query and checks
    size_t ws = 0;
    expect(mss_workspace_bytes(&d, MSS_OP_SELECTIVE_SCAN_BACKWARD, &ws), MSS_OK, "ws query");
    if (ws == 0) expect(1, 0, "ws query: nonzero size");
    expect(mss_workspace_bytes(&d, 99, &ws), MSS_EINVAL, "ws query: op");
    expect(mss_workspace_bytes(&huge, MSS_OP_SELECTIVE_SCAN_BACKWARD, &ws), MSS_EINVAL,
           "ws query: overflow");
    expect(mss_workspace_bytes(&d, MSS_OP_SELECTIVE_SCAN_BACKWARD, nullptr), MSS_EINVAL,
           "ws query: null out");
    size_t need = 0;
    mss_workspace_bytes(&d, MSS_OP_SELECTIVE_SCAN_BACKWARD, &need);
    expect(scan_bwd(&d, fake(7), fake(20), need - 1), MSS_EWORKSPACE, "scan bwd: small workspace");
    expect(scan_bwd(&d, fake(7), nullptr, need), MSS_EWORKSPACE, "scan bwd: null workspace");
    expect(scan_bwd(&d, fake(7), misaligned(20), need), MSS_EALIGN, "scan bwd: workspace align");
    expect(scan_bwd(&d, fake(1), fake(20), need), MSS_EALIAS, "scan bwd: du aliases u");
    expect(scan_bwd(&d, fake(7), fake(1), need), MSS_EALIAS, "scan bwd: workspace aliases u");
    mss_dims dck = d;
    dck.flags = MSS_FLAG_CKPT8;   // checkpoints announced but not given
    expect(scan_bwd(&dck, fake(7), fake(20), need), MSS_EINVAL, "scan bwd: CKPT8 without h_ckpt");
    size_t cneed = 0;
    expect(mss_workspace_bytes(&d, MSS_OP_CONV1D_SILU_BACKWARD, &cneed), MSS_OK, "conv ws query");
    expect(conv_bwd(&d, fake(1), fake(20), cneed), MSS_EALIAS, "conv bwd: dx aliases x");
    expect(conv_bwd(&d, fake(4), fake(20), 0), MSS_EWORKSPACE, "conv bwd: small workspace");
    expect(conv_bwd(&wide, fake(4), nullptr, 0), MSS_EINVAL, "conv bwd: D K overflow, L = 0");

    // Mamba-2 SSD
    mss_ssd_dims s2 = ssd_dims(2, 64, 8, 64, 128, 1);
    expect(ssd(nullptr, fake(1), fake(9)), MSS_EINVAL, "ssd: null dims");
    mss_ssd_dims sp = ssd_dims(2, 64, 8, 48, 128, 1);
    expect(ssd(&sp, fake(1), fake(9)), MSS_EINVAL, "ssd: head_dim 48");
    mss_ssd_dims sg = ssd_dims(2, 64, 8, 64, 128, 3);
    expect(ssd(&sg, fake(1), fake(9)), MSS_EINVAL, "ssd: groups");
    mss_ssd_dims sh = ssd_dims(big, big, 8, 64, 128, 1);
    expect(ssd(&sh, fake(1), fake(9)), MSS_EINVAL, "ssd: overflow");
    expect(ssd(&s2, fake(1), fake(1)), MSS_EALIAS, "ssd: y aliases x");
    expect(ssd(&s2, misaligned(1), fake(9)), MSS_EALIGN, "ssd: alignment");

    if (g_failed) {
        std::printf("%d check(s) failed\n", g_failed);
        return 1;
    }
    std::printf("all checks passed\n");
    return 0;
}
