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
#include <mutex>
#include <vector>

#include "launch.h"
#include "launch_bwd.h"
#include "launch_ssd.h"
#include "mss.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int32_t kKnownFlags = MSS_FLAG_EXACT | MSS_FLAG_CKPT8;   // every other bit is rejected

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
    if (!dims || dims->struct_size != static_cast<int32_t>(sizeof(mss_dims)) ||
        (dims->flags & ~kKnownFlags) != 0)
        return MSS_EINVAL;
    if (dims->batch < 0 || dims->d_inner < 0) return MSS_EINVAL;
    if (need_l && dims->seq_len < 0) return MSS_EINVAL;
    if (dims->d_state < 1 || dims->d_state > 16) return MSS_EINVAL;
    if (need_k && (dims->d_conv < 1 || dims->d_conv > 8)) return MSS_EINVAL;
    return MSS_OK;
}

// The time split.  Segment lengths depend on the problem shape alone (never
// on the device or the environment), so a call's output bits are a function
// of its inputs and shape.  The constants can be overridden at build time
// (-D...) for tuning experiments.
#ifndef MSS_SCAN_TARGET_WAVES
#define MSS_SCAN_TARGET_WAVES 2048   // two waves on each SIMD of a 256-CU MI355X
#endif
#ifndef MSS_SCAN_MIN_SEG
#define MSS_SCAN_MIN_SEG 64
#endif
#ifndef MSS_BWD_TARGET_WAVES
#define MSS_BWD_TARGET_WAVES 2048
#endif
#ifndef MSS_BWD_MIN_SEG
#define MSS_BWD_MIN_SEG 64
#endif
#ifndef MSS_SSD_TARGET_WG
#define MSS_SSD_TARGET_WG 1280       // five 4-wave workgroups per CU of 256
#endif
#ifndef MSS_SSD_MIN_SEG
#define MSS_SSD_MIN_SEG 64
#endif

bool exact(const mss_dims* dims) { return (dims->flags & MSS_FLAG_EXACT) != 0; }
bool ckpt8(const mss_dims* dims) { return (dims->flags & MSS_FLAG_CKPT8) != 0; }

// Segment length (steps of the flattened (tile, t) space) for `total` steps
// over tiles of L steps: equal segments for about `target` waves, none
// shorter than `min_seg`; MSS_FLAG_EXACT: one segment per tile.
int64_t split(int64_t total, int64_t L, int64_t target, int64_t min_seg, bool whole_tiles) {
    if (whole_tiles) return L > 0 ? L : 1;
    int64_t seg = (total + target - 1) / target;
    if (seg < min_seg) seg = min_seg;
    return seg < 1 ? 1 : seg;
}

mss::ScanShape scan_shape(const mss_dims* dims, const mss_strides& ld, const float* B,
                          const float* C, const float* z) {
    mss::ScanShape s;
    s.B = dims->batch;
    s.L = dims->seq_len;
    s.D = dims->d_inner;
    s.N = static_cast<int>(dims->d_state);
    s.K = static_cast<int>(dims->d_conv);
    s.tiles_per_b = (s.D + 63) / 64;
    s.Lp = (s.L + 7) / 8 * 8;
    s.total = s.B * s.tiles_per_b * s.Lp;
    s.seg = (split(s.total, s.Lp, MSS_SCAN_TARGET_WAVES, MSS_SCAN_MIN_SEG, exact(dims)) + 7) / 8 * 8;
    s.ld_src = ld.x;
    s.ld_z = ld.z;
    s.ld_delta = ld.delta;
    s.ld_B = ld.B;
    s.ld_C = ld.C;
    s.ld_y = ld.y;
    s.bc_vec = reinterpret_cast<uintptr_t>(B) % 16 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0 &&
               ld.B % 4 == 0 && ld.C % 4 == 0;
    // (the z stride matters only when z is given)
    s.dense = ld.x == s.D && (z == nullptr || ld.z == s.D) && ld.delta == s.D && ld.y == s.D &&
              ld.B == s.N && ld.C == s.N;
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
    int64_t M, MD, MN, DN, DK, BDN, BLDN;
    // h_cache: every step's state, or (MSS_FLAG_CKPT8) the state entering
    // every 8th step
    const int64_t Lc = ckpt8(dims) ? (L + 7) / 8 : L;
    if (!count(M, {Bt, L}) || !count(MD, {Bt, L, D}) || !count(MN, {Bt, L, N}) ||
        !count(DN, {D, N}) || !count(DK, {D, K}) || !count(BDN, {Bt, D, N}) ||
        (h_cache && !count(BLDN, {Bt, Lc, D, N})))
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
        ck.in(w_conv, DK, true);
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
    mss::ScanShape sh = scan_shape(dims, ld, B, C, z);
    sh.ckpt8 = ckpt8(dims);
    const hipError_t e = mss::launch_scan(a, sh, stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}

constexpr int64_t kBwdTile = 32;     // channels per wave in the scan backward
constexpr int64_t kBwdBlock = 8;     // steps per checkpointed block
constexpr int64_t kConvRun = 32;     // steps per job of the conv backward
constexpr int64_t kConvPartRows = 9; // kMaxK + 1

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Work split of the scan backward: the flattened (channel tile, t) space cut
// into segments of equal length, about two waves per SIMD, but no segment
// shorter than 64 steps: below that the two decay replays of a segment
// outweigh its own steps.
mss::BwdShape bwd_shape(const mss_dims* dims) {
    mss::BwdShape s;
    s.B = dims->batch;
    s.L = dims->seq_len;
    s.D = dims->d_inner;
    s.N = static_cast<int>(dims->d_state);
    s.tiles_per_b = (s.D + kBwdTile - 1) / kBwdTile;
    s.Lp = align_up(s.L, kBwdBlock);
    s.total = s.B * s.tiles_per_b * s.Lp;   // fits: B L D was counted without overflow
    const int64_t seg =
        align_up(split(s.total, s.Lp, MSS_BWD_TARGET_WAVES, MSS_BWD_MIN_SEG, exact(dims)), kBwdBlock);
    s.seg = seg;
    s.waves = (s.total + seg - 1) / seg;
    s.blocks_per_seg = (seg + kBwdBlock - 1) / kBwdBlock;
    // a tile of Lp steps meets at most ceil(Lp / seg) + 1 segments
    s.pieces = (s.Lp + seg - 1) / seg + 1;
    s.bc_vec = false;
    return s;
}

// Byte offsets of the workspace regions of the scan backward.
struct BwdLayout {
    int64_t ckpt, partB, partC, partA, partD, total;
};

// with_ckpt false: the forward's checkpoints are given and the checkpoint
// region is not needed.
bool bwd_layout(const mss::BwdShape& s, BwdLayout& o, bool with_ckpt) {
    int64_t ck, pb, pa, pd;
    if (!count(ck, {with_ckpt ? s.waves : 0, s.blocks_per_seg, 64 * 8 * 4}) ||
        !count(pb, {s.B, s.tiles_per_b, s.L, 16 * 4}) ||
        !count(pa, {s.B, s.tiles_per_b, s.pieces, 64 * 8 * 4}) ||
        !count(pd, {s.B, s.tiles_per_b, s.pieces, 32 * 4}))
        return false;
    o.ckpt = 0;
    o.partB = align_up(o.ckpt + ck, 256);
    o.partC = align_up(o.partB + pb, 256);
    o.partA = align_up(o.partC + pb, 256);
    o.partD = align_up(o.partA + pa, 256);
    o.total = align_up(o.partD + pd, 256);
    return true;
}

int64_t conv_bwd_groups(const mss_dims* dims) {
    const int64_t tiles = (dims->d_inner + 63) / 64;
    const int64_t jobs = dims->batch * ((dims->seq_len + kConvRun - 1) / kConvRun);
    const int64_t target = MSS_BWD_TARGET_WAVES;   // fixed: the dw, db summation order depends on it
    int64_t g = tiles > 0 ? (target + tiles - 1) / tiles : 1;
    if (g > jobs) g = jobs;
    if (g < 1) g = 1;
    return g;
}

int64_t conv_bwd_bytes(const mss_dims* dims) {
    const int64_t tiles = (dims->d_inner + 63) / 64;
    return align_up(tiles * conv_bwd_groups(dims) * kConvPartRows * 64 * 4, 256);
}

int check_workspace(void* ws, size_t bytes, int64_t need) {
    if (need == 0) return MSS_OK;
    if (!ws || static_cast<int64_t>(bytes) < need) return MSS_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MSS_EALIGN;
    return MSS_OK;
}

int zero_fill(float* p, int64_t n, hipStream_t stream) {
    if (!p || n <= 0) return MSS_OK;
    const hipError_t e = mss::launch_state_init(nullptr, p, n, stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}

bool ssd_dims_ok(const mss_ssd_dims* dims) {
    return dims && dims->struct_size == static_cast<int32_t>(sizeof(mss_ssd_dims)) &&
           (dims->flags & ~kKnownFlags) == 0;
}

// SSD segments per (batch row, head): about MSS_SSD_TARGET_WG workgroups in
// all (three are resident per CU at a time for the common shapes),
// none shorter than MSS_SSD_MIN_SEG steps (two chunks), so that the replay
// that rebuilds a segment's initial state does not outweigh its own steps;
// then rounded so that every segment has the same number of chunks.
int64_t ssd_segments(int64_t bh, int64_t nchunks, bool whole) {
    if (whole || bh <= 0 || nchunks <= 0) return 1;
    const int64_t Q = mss::ssd_chunk_len();
    int64_t nseg = MSS_SSD_TARGET_WG / bh;
    const int64_t min_chunks = (MSS_SSD_MIN_SEG + Q - 1) / Q;
    const int64_t max_seg = (nchunks + min_chunks - 1) / min_chunks;
    if (nseg > max_seg) nseg = max_seg;
    if (nseg < 1) nseg = 1;
    const int64_t seg_chunks = (nchunks + nseg - 1) / nseg;
    return (nchunks + seg_chunks - 1) / seg_chunks;
}

}  // namespace

// ---- the static scratch array of mss_selective_scan_backward_noalloc -------
// For callers that cannot allocate (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the scan backward's workspace in a
// device array of the library itself.  Each GPU the library runs on holds
// its own copy from the time the code object is loaded until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is taken once per device, with that device
// current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = static_cast<size_t>(MSS_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return MSS_EINVAL;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e);
            if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return MSS_EHIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MSS_OK;
}

// The scan backward with its workspace from the caller (use_scratch false) or
// from the library's static scratch array (use_scratch true; workspace is
// then ignored).
int scan_bwd_common(const mss_dims* dims, int disc, const float* u, const float* delta,
                    const float* A_log, const float* B, const float* C, const float* D_vec,
                    const float* z, const float* h0, const float* h_ckpt, const float* dout, float* du,
                    float* ddelta, float* dA_log, float* dB, float* dC, float* dD_vec, float* dz,
                    float* dh0, bool use_scratch, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    int st = check_dims(dims, true, false);
    if (st != MSS_OK) return st;
    if (disc != MSS_DISC_ZOH && disc != MSS_DISC_EULER) return MSS_EINVAL;
    const int64_t Bt = dims->batch, L = dims->seq_len, D = dims->d_inner, N = dims->d_state;
    int64_t MD, MN, DN, BDN;
    if (!count(MD, {Bt, L, D}) || !count(MN, {Bt, L, N}) || !count(DN, {D, N}) ||
        !count(BDN, {Bt, D, N}))
        return MSS_EINVAL;
    if (z && !dz && MD > 0) return MSS_EINVAL;
    // MSS_FLAG_CKPT8 and h_ckpt go together (the flag sizes the workspace)
    const bool with_ck = ckpt8(dims);
    if (with_ck != (h_ckpt != nullptr) && MD > 0) return MSS_EINVAL;
    int64_t BKDN = 0;
    if (with_ck && !count(BKDN, {Bt, (L + 7) / 8, D, N})) return MSS_EINVAL;
    Checker ck;
    ck.in(u, MD, true);
    ck.in(h_ckpt, BKDN, false);
    ck.in(delta, MD, true);
    ck.in(A_log, DN, true);
    ck.in(B, MN, true);
    ck.in(C, MN, true);
    ck.in(D_vec, D, false);
    ck.in(z, MD, false);
    ck.in(h0, BDN, false);
    ck.in(dout, MD, true);
    ck.out(du, MD, true);
    ck.out(ddelta, MD, true);
    ck.out(dA_log, DN, true);
    ck.out(dB, MN, true);
    ck.out(dC, MN, true);
    ck.out(dD_vec, D, false);
    ck.out(dz, z ? MD : 0, false);
    ck.out(dh0, BDN, false);
    int64_t need = 0;
    mss::BwdShape s{};
    BwdLayout lay{};
    if (MD > 0) {
        s = bwd_shape(dims);
        if (!bwd_layout(s, lay, !with_ck)) return MSS_EINVAL;
        if (s.waves > INT32_MAX) return MSS_EINVAL;   // grid size
        need = lay.total;
    }
    // The workspace is an output like the others: it may not overlap anything.
    if (!use_scratch && need > 0 && workspace) ck.outs.push_back({workspace, need});
    st = ck.finish();
    if (st != MSS_OK) return st;
    if (use_scratch) {
        // checked before any HIP call: a request past the static array's size
        // is refused without touching the device
        if (need > static_cast<int64_t>(kScratchBytes)) return MSS_ESCRATCH;
        if (need > 0) {
            st = scratch_address(&workspace);
            if (st != MSS_OK) return st;
            workspace_bytes = kScratchBytes;
        }
    } else {
        st = check_workspace(workspace, workspace_bytes, need);
        if (st != MSS_OK) return st;
    }
    if (MD == 0) {
        // Nothing depends on the parameters: their gradients are zero.
        if ((st = zero_fill(dA_log, DN, stream)) != MSS_OK) return st;
        if ((st = zero_fill(dD_vec, D, stream)) != MSS_OK) return st;
        return zero_fill(dh0, BDN, stream);
    }
    s.bc_vec = N == 16 && reinterpret_cast<uintptr_t>(B) % 16 == 0 &&
               reinterpret_cast<uintptr_t>(C) % 16 == 0;
    char* w = static_cast<char*>(workspace);
    const mss::BwdArgs a{disc, u, delta, A_log, B, C, D_vec, z, h0, with_ck ? h_ckpt : nullptr,
                         dout, du, ddelta, dA_log,
                         dB, dC, dD_vec, z ? dz : nullptr, dh0,
                         reinterpret_cast<float*>(w + lay.ckpt),
                         reinterpret_cast<float*>(w + lay.partB),
                         reinterpret_cast<float*>(w + lay.partC),
                         reinterpret_cast<float*>(w + lay.partA),
                         reinterpret_cast<float*>(w + lay.partD)};
    const hipError_t e = mss::launch_scan_bwd(a, s, stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int mss_time_split(const mss_dims* dims, int op, int64_t* segment_steps) {
    if (!segment_steps) return MSS_EINVAL;
    *segment_steps = 0;
    const int st = check_dims(dims, true, false);
    if (st != MSS_OK) return st;
    int64_t MD;
    if (!count(MD, {dims->batch, dims->seq_len, dims->d_inner})) return MSS_EINVAL;
    if (op == MSS_OP_SELECTIVE_SCAN) {
        const mss_strides ld = dense_strides(dims);
        *segment_steps = MD > 0 ? scan_shape(dims, ld, nullptr, nullptr, nullptr).seg : 0;
        return MSS_OK;
    }
    if (op == MSS_OP_SELECTIVE_SCAN_BACKWARD) {
        *segment_steps = MD > 0 ? bwd_shape(dims).seg : 0;
        return MSS_OK;
    }
    return MSS_EINVAL;
}

int mss_ssd_time_split(const mss_ssd_dims* dims, int64_t* segment_steps) {
    if (!segment_steps) return MSS_EINVAL;
    *segment_steps = 0;
    if (!ssd_dims_ok(dims) || dims->batch < 0 || dims->seq_len < 0 || dims->n_heads < 1)
        return MSS_EINVAL;
    int64_t bh;
    if (!count(bh, {dims->batch, dims->n_heads})) return MSS_EINVAL;
    if (bh == 0 || dims->seq_len == 0) return MSS_OK;
    const int64_t Q = mss::ssd_chunk_len();
    const int64_t nchunks = (dims->seq_len + Q - 1) / Q;
    const int64_t nseg = ssd_segments(bh, nchunks, (dims->flags & MSS_FLAG_EXACT) != 0);
    *segment_steps = (nchunks + nseg - 1) / nseg * Q;
    return MSS_OK;
}

int mss_workspace_bytes(const mss_dims* dims, int op, size_t* bytes) {
    if (!bytes) return MSS_EINVAL;
    *bytes = 0;
    if (op == MSS_OP_SELECTIVE_SCAN_BACKWARD) {
        int st = check_dims(dims, true, false);
        if (st != MSS_OK) return st;
        int64_t MD;
        if (!count(MD, {dims->batch, dims->seq_len, dims->d_inner})) return MSS_EINVAL;
        if (MD == 0) return MSS_OK;
        BwdLayout lay;
        if (!bwd_layout(bwd_shape(dims), lay, !ckpt8(dims))) return MSS_EINVAL;
        *bytes = static_cast<size_t>(lay.total);
        return MSS_OK;
    }
    if (op == MSS_OP_CONV1D_SILU_BACKWARD) {
        int st = check_dims(dims, true, true);
        if (st != MSS_OK) return st;
        int64_t MD;
        if (!count(MD, {dims->batch, dims->seq_len, dims->d_inner})) return MSS_EINVAL;
        if (MD == 0) return MSS_OK;
        *bytes = static_cast<size_t>(conv_bwd_bytes(dims));
        return MSS_OK;
    }
    return MSS_EINVAL;
}

int mss_selective_scan_backward(const mss_dims* dims, int disc, const float* u,
                                const float* delta, const float* A_log, const float* B,
                                const float* C, const float* D_vec, const float* z,
                                const float* h0, const float* h_ckpt, const float* dout,
                                float* du, float* ddelta, float* dA_log, float* dB, float* dC,
                                float* dD_vec, float* dz, float* dh0, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    return scan_bwd_common(dims, disc, u, delta, A_log, B, C, D_vec, z, h0, h_ckpt, dout, du, ddelta,
                           dA_log, dB, dC, dD_vec, dz, dh0, false, workspace, workspace_bytes,
                           stream);
}

int mss_selective_scan_backward_noalloc(const mss_dims* dims, int disc, const float* u,
                                        const float* delta, const float* A_log, const float* B,
                                        const float* C, const float* D_vec, const float* z,
                                        const float* h0, const float* h_ckpt, const float* dout,
                                        float* du, float* ddelta, float* dA_log, float* dB,
                                        float* dC, float* dD_vec, float* dz, float* dh0,
                                        hipStream_t stream) {
    return scan_bwd_common(dims, disc, u, delta, A_log, B, C, D_vec, z, h0, h_ckpt, dout, du, ddelta,
                           dA_log, dB, dC, dD_vec, dz, dh0, true, nullptr, 0, stream);
}

int mss_conv1d_silu_backward(const mss_dims* dims, const float* x, const float* w_conv,
                             const float* b_conv, const float* du, float* dx, float* dw_conv,
                             float* db_conv, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    int st = check_dims(dims, true, true);
    if (st != MSS_OK) return st;
    const int64_t Bt = dims->batch, L = dims->seq_len, D = dims->d_inner, K = dims->d_conv;
    int64_t MD, DK;
    if (!count(MD, {Bt, L, D}) || !count(DK, {D, K})) return MSS_EINVAL;
    Checker ck;
    ck.in(x, MD, true);
    ck.in(w_conv, DK, true);
    ck.in(b_conv, D, false);
    ck.in(du, MD, true);
    ck.out(dx, MD, true);
    ck.out(dw_conv, DK, true);
    ck.out(db_conv, D, false);
    const int64_t need = MD > 0 ? conv_bwd_bytes(dims) : 0;
    if (MD > 0 && ((D + 63) / 64) * conv_bwd_groups(dims) > INT32_MAX) return MSS_EINVAL;
    if (need > 0 && workspace) ck.outs.push_back({workspace, need});
    st = ck.finish();
    if (st != MSS_OK) return st;
    st = check_workspace(workspace, workspace_bytes, need);
    if (st != MSS_OK) return st;
    if (MD == 0) {
        if ((st = zero_fill(dw_conv, DK, stream)) != MSS_OK) return st;
        return zero_fill(db_conv, D, stream);
    }
    const mss::ConvBwdArgs a{Bt, L, D, static_cast<int>(K), conv_bwd_groups(dims), x, w_conv,
                             b_conv, du, dx, dw_conv, db_conv, static_cast<float*>(workspace)};
    const hipError_t e = mss::launch_conv1d_silu_bwd(a, stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}


int mss_conv1d_silu(const mss_dims* dims, const float* x, const float* w_conv, const float* b_conv,
                    float* u, hipStream_t stream) {
    int st = check_dims(dims, true, true);
    if (st != MSS_OK) return st;
    const int64_t Bt = dims->batch, L = dims->seq_len, D = dims->d_inner, K = dims->d_conv;
    int64_t MD, DK;
    if (!count(MD, {Bt, L, D}) || !count(DK, {D, K})) return MSS_EINVAL;
    Checker ck;
    ck.in(x, MD, true);
    ck.in(w_conv, DK, true);
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
    int64_t BD, BN, DN, DK, BDN, BKD;
    if (!count(BD, {Bt, D}) || !count(BN, {Bt, N}) || !count(DN, {D, N}) ||
        !count(DK, {D, K}) || !count(BDN, {Bt, D, N}) || !count(BKD, {Bt, K - 1, D}))
        return MSS_EINVAL;
    Checker ck;
    ck.in(x, BD, true);
    ck.in(z, BD, false);
    ck.in(delta, BD, true);
    ck.in(A_log, DN, true);
    ck.in(B, BN, true);
    ck.in(C, BN, true);
    ck.in(D_vec, D, false);
    ck.in(w_conv, DK, true);
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

int mss_ssd_scan(const mss_ssd_dims* dims, int disc, const float* x, const float* dt, const float* A_log,
                 const float* B, const float* C, const float* D_vec, const float* dt_bias,
                 const float* h0, float* y, float* h_last, hipStream_t stream) {
    if (!ssd_dims_ok(dims)) return MSS_EINVAL;
    const int64_t Bt = dims->batch, L = dims->seq_len, H = dims->n_heads, P = dims->head_dim;
    const int64_t N = dims->d_state, G = dims->n_groups;
    if (Bt < 0 || L < 0 || H < 1 || G < 1 || H % G != 0 || !mss::ssd_supported(P, N))
        return MSS_EINVAL;
    if (disc != MSS_DISC_ZOH && disc != MSS_DISC_EULER) return MSS_EINVAL;
    int64_t M, MHP, MH, MGN, BHPN;
    if (!count(M, {Bt, L}) || !count(MHP, {Bt, L, H, P}) || !count(MH, {Bt, L, H}) ||
        !count(MGN, {Bt, L, G, N}) || !count(BHPN, {Bt, H, P, N}))
        return MSS_EINVAL;
    Checker ck;
    ck.in(x, MHP, true);
    ck.in(dt, MH, true);
    ck.in(A_log, H, true);
    ck.in(B, MGN, true);
    ck.in(C, MGN, true);
    ck.in(D_vec, H, false);
    ck.in(dt_bias, H, false);
    ck.in(h0, BHPN, false);
    ck.out(y, MHP, true);
    ck.out(h_last, BHPN, false);
    int st = ck.finish();
    if (st != MSS_OK) return st;
    if (Bt == 0) return MSS_OK;
    if (L == 0) {
        if (!h_last) return MSS_OK;
        const hipError_t e = mss::launch_state_init(h0, h_last, BHPN, stream);
        return e == hipSuccess ? MSS_OK : hip_fail(e);
    }
    const int64_t Q = mss::ssd_chunk_len();
    const int64_t nchunks = (L + Q - 1) / Q;
    const int64_t nseg = ssd_segments(Bt * H, nchunks, (dims->flags & MSS_FLAG_EXACT) != 0);
    const int64_t bh = Bt * H;
    const int64_t seg_chunks = (nchunks + nseg - 1) / nseg;
    if (bh * nseg > INT32_MAX) return MSS_EINVAL;
    const mss::SsdArgs a{disc, Bt, L, H, P, N, G, nseg, seg_chunks, x, dt, A_log, B, C,
                         D_vec, dt_bias, h0, y, h_last};
    const hipError_t e = mss::launch_ssd(a, stream);
    return e == hipSuccess ? MSS_OK : hip_fail(e);
}

const char* mss_strerror(int status) {
    switch (status) {
        case MSS_OK: return "ok";
        case MSS_EINVAL: return "invalid argument (null tensor, size out of range, bad struct_size or disc)";
        case MSS_EALIGN: return "pointer not 16-byte aligned";
        case MSS_EALIAS: return "an output overlaps an input or another output";
        case MSS_EWORKSPACE: return "workspace missing or smaller than mss_workspace_bytes reports";
        case MSS_EHIP: return "HIP runtime error (see mss_last_hip_error)";
        case MSS_ESCRATCH: return "the problem needs more scratch than the library's static "
                                  "array holds (MSS_NOALLOC_SCRATCH_BYTES); use the entry point "
                                  "with a caller workspace";
        default: return "unknown status";
    }
}

int mss_version(void) { return MSS_VERSION; }

int mss_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
