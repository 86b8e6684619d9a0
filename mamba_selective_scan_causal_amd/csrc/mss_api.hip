// mss_api.hip -- the extern "C" entry points of libmss: argument validation,
// work-split selection and kernel dispatch on the caller's stream.
//
// Validation follows the pages' rule of failing loudly on a wrong-size or
// missing tensor instead of computing garbage (builderforce-memory-engine
// 2026.7.14 -> 2026.9.28, dist/training/model_cpu.js, cpuWeightsFromNamed),
// and guards the parameter-block size the way the ConvParams fix in
// src/model/mamba1_block.ts calls for (a struct of the wrong size is rejected).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "launch.h"
#include "mss.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = static_cast<int>(e);
    return MSS_EHIP;
}

struct Span {
    const void* p;
    int64_t bytes;
};

bool overlap(const Span& a, const Span& b) {
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

// n1 * n2 * ... with overflow detection (all factors >= 0).
bool mul_ok(int64_t& acc, int64_t f) {
    if (f == 0 || acc == 0) {
        acc = 0;
        return true;
    }
    if (acc > INT64_MAX / f) return false;
    acc *= f;
    return true;
}

bool count(int64_t& out, std::initializer_list<int64_t> fs) {
    int64_t acc = 1;
    for (int64_t f : fs)
        if (!mul_ok(acc, f)) return false;
    if (acc > INT64_MAX / 16) return false;  // byte offsets (x4) plus headroom
    out = acc;
    return true;
}

struct Checker {
    int status = MSS_OK;
    std::vector<Span> ins, outs;

    // A dense tensor of `elems` fp32 values (16-byte aligned).  Required
    // tensors may be NULL only when they hold no elements.
    void in(const float* p, int64_t elems, bool required) { add(ins, p, elems * 4, required, 16); }
    void out(float* p, int64_t elems, bool required) { add(outs, p, elems * 4, required, 16); }
    // `rows` rows of `width` fp32 values, row r at p + r * stride (4-byte aligned).
    void in_rows(const float* p, int64_t rows, int64_t width, int64_t stride, bool required) {
        add(ins, p, rows_bytes(rows, width, stride), required, 4);
    }
    void out_rows(float* p, int64_t rows, int64_t width, int64_t stride, bool required) {
        add(outs, p, rows_bytes(rows, width, stride), required, 4);
    }

    int64_t rows_bytes(int64_t rows, int64_t width, int64_t stride) {
        if (rows <= 0 || width <= 0) return 0;
        int64_t span;
        if (stride < width || !count(span, {rows - 1, stride}) || span > INT64_MAX / 8 - width) {
            if (status == MSS_OK) status = MSS_EINVAL;
            return 0;
        }
        return (span + width) * 4;
    }

    void add(std::vector<Span>& v, const void* p, int64_t bytes, bool required, uintptr_t align) {
        if (status != MSS_OK) return;
        if (!p) {
            if (required && bytes > 0) status = MSS_EINVAL;
            return;
        }
        if (reinterpret_cast<uintptr_t>(p) % align != 0) {
            status = MSS_EALIGN;
            return;
        }
        v.push_back({p, bytes});
    }

    int finish() {
        if (status != MSS_OK) return status;
        for (size_t i = 0; i < outs.size(); i++) {
            for (const Span& s : ins)
                if (overlap(outs[i], s)) return MSS_EALIAS;
            for (size_t j = i + 1; j < outs.size(); j++)
                if (overlap(outs[i], outs[j])) return MSS_EALIAS;
        }
        return MSS_OK;
    }
};

int check_dims(const mss_dims* dims, bool need_l, bool need_k) {
    if (!dims || dims->struct_size != static_cast<int32_t>(sizeof(mss_dims)) || dims->reserved != 0)
        return MSS_EINVAL;
    if (dims->batch < 0 || dims->d_inner < 0) return MSS_EINVAL;
    if (need_l && dims->seq_len < 0) return MSS_EINVAL;
    if (dims->d_state < 1 || dims->d_state > 16) return MSS_EINVAL;
    if (need_k && (dims->d_conv < 1 || dims->d_conv > 8)) return MSS_EINVAL;
    return MSS_OK;
}

// Waves per CU for the scan (2 per SIMD) and the shortest segment; both can
// be overridden through the environment for tuning experiments.
int64_t env_or(const char* name, int64_t dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    const long long x = std::atoll(v);
    return x > 0 ? x : dflt;
}

int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev < 0 || dev >= 64) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

mss::ScanShape scan_shape(const mss_dims* dims, const mss_strides& ld, const float* B,
                          const float* C) {
    static const int64_t waves_per_cu = env_or("MSS_SCAN_WAVES_PER_CU", 8);
    static const int64_t min_seg = env_or("MSS_SCAN_MIN_SEG", 512);
    mss::ScanShape s;
    s.B = dims->batch;
    s.L = dims->seq_len;
    s.D = dims->d_inner;
    s.N = static_cast<int>(dims->d_state);
    s.K = static_cast<int>(dims->d_conv);
    s.tiles_per_b = (s.D + 63) / 64;
    s.total = s.B * s.tiles_per_b * s.L;
    const int64_t target = cu_count() * waves_per_cu;
    int64_t seg = (s.total + target - 1) / target;
    if (seg < min_seg) seg = min_seg;
    s.seg = seg;
    s.ld_src = ld.x;
    s.ld_z = ld.z;
    s.ld_delta = ld.delta;
    s.ld_B = ld.B;
    s.ld_C = ld.C;
    s.ld_y = ld.y;
    s.bc_vec = reinterpret_cast<uintptr_t>(B) % 16 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0 &&
               ld.B % 4 == 0 && ld.C % 4 == 0;
    s.dense = ld.x == s.D && ld.z == s.D && ld.delta == s.D && ld.y == s.D && ld.B == s.N &&
              ld.C == s.N;
    return s;
}

mss_strides dense_strides(const mss_dims* dims) {
    mss_strides s;
    s.struct_size = sizeof(mss_strides);
    s.reserved = 0;
    s.x = s.z = s.delta = s.y = dims->d_inner;
    s.B = s.C = dims->d_state;
    return s;
}

// strided: the caller's strides (activations and B/C may be 4-byte aligned
// column slices); otherwise dense tensors with the 16-byte rule everywhere.
int scan_common(const mss_dims* dims, const mss_strides* strides, bool strided, int disc,
                bool fused, const float* src, const float* w_conv, const float* b_conv,
                const float* delta, const float* A_log, const float* B, const float* C,
                const float* D_vec, const float* z, const float* h0, float* y, float* h_cache,
                float* h_last, hipStream_t stream) {
    int st = check_dims(dims, true, fused);
    if (st != MSS_OK) return st;
    if (disc != MSS_DISC_ZOH && disc != MSS_DISC_EULER) return MSS_EINVAL;
    if (strided && (!strides || strides->struct_size != static_cast<int32_t>(sizeof(mss_strides)) ||
                    strides->reserved != 0))
        return MSS_EINVAL;
    const mss_strides ld = strided ? *strides : dense_strides(dims);
    const int64_t Bt = dims->batch, L = dims->seq_len, D = dims->d_inner, N = dims->d_state;
    const int64_t K = dims->d_conv;
    int64_t M, MD, MN, DN, BDN, BLDN;
    if (!count(M, {Bt, L}) || !count(MD, {Bt, L, D}) || !count(MN, {Bt, L, N}) ||
        !count(DN, {D, N}) || !count(BDN, {Bt, D, N}) ||
        (h_cache && !count(BLDN, {Bt, L, D, N})))
        return MSS_EINVAL;
    if (!h_cache) BLDN = 0;
    Checker ck;
    if (strided) {
        ck.in_rows(src, M, D, ld.x, true);
        ck.in_rows(delta, M, D, ld.delta, true);
        ck.in_rows(B, M, N, ld.B, true);
        ck.in_rows(C, M, N, ld.C, true);
        ck.in_rows(z, M, D, ld.z, false);
        ck.out_rows(y, M, D, ld.y, true);
    } else {
        ck.in(src, MD, true);
        ck.in(delta, MD, true);
        ck.in(B, MN, true);
        ck.in(C, MN, true);
        ck.in(z, MD, false);
        ck.out(y, MD, true);
    }
    if (fused) {
        ck.in(w_conv, D * K, true);
        ck.in(b_conv, D, false);
    }
    ck.in(A_log, DN, true);
    ck.in(D_vec, D, false);
    ck.in(h0, BDN, false);
    ck.out(h_cache, BLDN, false);
    ck.out(h_last, BDN, false);
    st = ck.finish();
    if (st != MSS_OK) return st;
    if (Bt == 0 || D == 0) return MSS_OK;
    if (L == 0) {
        if (!h_last) return MSS_OK;
        const hipError_t e = mss::launch_state_init(h0, h_last, BDN, stream);
        return e == hipSuccess ? MSS_OK : hip_fail(e);
    }
    const mss::ScanArgs a{disc, fused, src, delta, A_log, B, C, D_vec, z, h0, w_conv, b_conv,
                          y, h_cache, h_last};
    const hipError_t e = mss::launch_scan(a, scan_shape(dims, ld, B, C), stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int mss_conv1d_silu(const mss_dims* dims, const float* x, const float* w_conv, const float* b_conv,
                    float* u, hipStream_t stream) {
    int st = check_dims(dims, true, true);
    if (st != MSS_OK) return st;
    const int64_t Bt = dims->batch, L = dims->seq_len, D = dims->d_inner, K = dims->d_conv;
    int64_t MD;
    if (!count(MD, {Bt, L, D})) return MSS_EINVAL;
    Checker ck;
    ck.in(x, MD, true);
    ck.in(w_conv, D * K, true);
    ck.in(b_conv, D, false);
    ck.out(u, MD, true);
    st = ck.finish();
    if (st != MSS_OK) return st;
    if (MD == 0) return MSS_OK;
    const mss::ConvArgs a{Bt, L, D, static_cast<int>(K), x, w_conv, b_conv, u};
    const hipError_t e = mss::launch_conv1d_silu(a, stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}

int mss_selective_scan(const mss_dims* dims, int disc, const float* u, const float* delta,
                       const float* A_log, const float* B, const float* C, const float* D_vec,
                       const float* z, const float* h0, float* y, float* h_cache, float* h_last,
                       hipStream_t stream) {
    return scan_common(dims, nullptr, false, disc, false, u, nullptr, nullptr, delta, A_log, B,
                       C, D_vec, z, h0, y, h_cache, h_last, stream);
}

int mss_selective_scan_strided(const mss_dims* dims, const mss_strides* strides, int disc,
                               const float* u, const float* delta, const float* A_log,
                               const float* B, const float* C, const float* D_vec,
                               const float* z, const float* h0, float* y, float* h_cache,
                               float* h_last, hipStream_t stream) {
    return scan_common(dims, strides, true, disc, false, u, nullptr, nullptr, delta, A_log, B,
                       C, D_vec, z, h0, y, h_cache, h_last, stream);
}

int mss_mamba1_core(const mss_dims* dims, int disc, const float* x, const float* w_conv,
                    const float* b_conv, const float* delta, const float* A_log, const float* B,
                    const float* C, const float* D_vec, const float* z, const float* h0, float* y,
                    float* h_cache, float* h_last, hipStream_t stream) {
    return scan_common(dims, nullptr, false, disc, true, x, w_conv, b_conv, delta, A_log, B, C,
                       D_vec, z, h0, y, h_cache, h_last, stream);
}

int mss_mamba1_core_strided(const mss_dims* dims, const mss_strides* strides, int disc,
                            const float* x, const float* w_conv, const float* b_conv,
                            const float* delta, const float* A_log, const float* B,
                            const float* C, const float* D_vec, const float* z,
                            const float* h0, float* y, float* h_cache, float* h_last,
                            hipStream_t stream) {
    return scan_common(dims, strides, true, disc, true, x, w_conv, b_conv, delta, A_log, B, C,
                       D_vec, z, h0, y, h_cache, h_last, stream);
}

int mss_selective_step(const mss_dims* dims, int disc, const float* x, const float* z,
                       const float* delta, const float* A_log, const float* B, const float* C,
                       const float* D_vec, const float* w_conv, const float* b_conv,
                       float* conv_state, float* h, float* y, hipStream_t stream) {
    int st = check_dims(dims, false, true);
    if (st != MSS_OK) return st;
    if (disc != MSS_DISC_ZOH && disc != MSS_DISC_EULER) return MSS_EINVAL;
    const int64_t Bt = dims->batch, D = dims->d_inner, N = dims->d_state, K = dims->d_conv;
    int64_t BD, BN, DN, BDN, BKD;
    if (!count(BD, {Bt, D}) || !count(BN, {Bt, N}) || !count(DN, {D, N}) ||
        !count(BDN, {Bt, D, N}) || !count(BKD, {Bt, K - 1, D}))
        return MSS_EINVAL;
    Checker ck;
    ck.in(x, BD, true);
    ck.in(z, BD, false);
    ck.in(delta, BD, true);
    ck.in(A_log, DN, true);
    ck.in(B, BN, true);
    ck.in(C, BN, true);
    ck.in(D_vec, D, false);
    ck.in(w_conv, D * K, true);
    ck.in(b_conv, D, false);
    ck.out(conv_state, BKD, true);
    ck.out(h, BDN, true);
    ck.out(y, BD, true);
    st = ck.finish();
    if (st != MSS_OK) return st;
    if (BD == 0) return MSS_OK;
    const mss::StepArgs a{disc, Bt, D, static_cast<int>(N), static_cast<int>(K), x, z, delta,
                          A_log, B, C, D_vec, w_conv, b_conv, conv_state, h, y};
    const hipError_t e = mss::launch_step(a, stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}

const char* mss_strerror(int status) {
    switch (status) {
        case MSS_OK: return "ok";
        case MSS_EINVAL: return "invalid argument (null tensor, size out of range, bad struct_size or disc)";
        case MSS_EALIGN: return "pointer not 16-byte aligned";
        case MSS_EALIAS: return "an output overlaps an input or another output";
        case MSS_EHIP: return "HIP runtime error (see mss_last_hip_error)";
        default: return "unknown status";
    }
}

int mss_version(void) { return MSS_VERSION; }

int mss_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
