/*
 * mss.h -- C ABI of libmss: the data-parallel core of a Mamba-1 (S6) block on
 * AMD Instinct MI355X (gfx950), hand-written HIP.
 *
 * The operation is the one the pages of the npm package
 * "@seanhogg/builderforce-memory-engine" define in the diff
 * 2026.7.12 -> 2026.9.27, file src/training/mamba1_cpu.ts, function
 * mamba1CpuForward, steps 4 (causal depthwise conv1d), 5 (SiLU), 8 (selective
 * scan with softplus(delta), A = -exp(clamp(A_log, -10, 5)), exponential
 * discretisation, recurrence, y = sum_n C h + D u) and 9 (gate by SiLU(z)),
 * with the layouts listed in that file's header comment.  The GPU dispatch
 * of the same computation (conv1d_forward, forward_scan, forward_reduce and
 * the h_cache binding) is in the diff 2026.7.14 -> 2026.9.28, file
 * src/model/mamba1_block.ts, Mamba1Block.forward.
 *
 * Symbols: B = batch, L = seq_len, M = B * L, D = d_inner, N = d_state,
 * K = d_conv.  Row r = b * L + t.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers to dense, row-major fp32 arrays
 *     on the current HIP device, allocated and owned by the caller.  The
 *     library allocates nothing and never frees a caller buffer; the backward
 *     passes take a caller workspace.  Its only device state is the static
 *     scratch array of mss_selective_scan_backward_noalloc.
 *   - Every pointer must be 16-byte aligned (MSS_EALIGN otherwise), except
 *     the activation and B/C tensors of the *_strided entry points (4 bytes).
 *   - Outputs may not overlap any input (MSS_EALIAS), except the state
 *     buffers of mss_selective_step, which are updated in place by design.
 *   - Work is enqueued on `stream` (NULL = the null stream) and the call
 *     returns without synchronising.  Arguments are validated before any
 *     launch; a call that returns an error has written nothing.
 *   - A zero size (B, L or D = 0) is valid and launches nothing, except that
 *     a sequence of length 0 still defines h_last (= h0, or zeros).
 *   - Limits: 1 <= N <= 16; 1 <= K <= 8.  Dimensions are int64; element
 *     offsets are computed in 64 bits.
 *   - NaN or Inf inputs are outside the contract: the kernels terminate and
 *     write every output, but the values are unspecified.
 *   - Calls on different streams may run concurrently; they share nothing.
 */
#ifndef MSS_H
#define MSS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSS_VERSION 2

/* Status codes. */
#define MSS_OK 0
#define MSS_EINVAL (-1)     /* null required pointer, bad size or limit, bad struct_size, bad disc */
#define MSS_EALIGN (-2)     /* a pointer is not 16-byte aligned */
#define MSS_EALIAS (-3)     /* an output overlaps an input */
#define MSS_EWORKSPACE (-4) /* workspace NULL or smaller than mss_workspace_bytes */
#define MSS_EHIP (-5)       /* a HIP runtime call or kernel launch failed; see mss_last_hip_error */
#define MSS_ESCRATCH (-6)   /* needs more than MSS_NOALLOC_SCRATCH_BYTES (the *_noalloc entry point) */

/* Problem sizes.  `struct_size` must be sizeof(mss_dims): it guards against a
 * caller built against a different layout of this struct.
 *
 * Time split.  The recurrence of every (b, d) column runs sequentially in
 * time, and a Mamba-1 problem has few enough columns that the scans split
 * time into segments processed in parallel.  A segment that starts at
 * t0 > 0 rebuilds the state it starts from, h(t0-1), by replaying the
 * recurrence from h = 0 over a window [tw, t0): tw is the latest step from
 * which every state of the segment's columns has decayed by at least
 * 2^-MSS_REPLAY_DECAY_BITS (prod aBar = exp(A sum dv), decided from delta
 * alone), or tw = 0.  (A state that decays faster than the slowest one
 * joins the replay later, at the 8-step block from which its own decay
 * reaches the same bound.)  Relative to the plain sequential recurrence the
 * state at t >= t0 then lacks exactly
 *     prod_{s=tj..t} aBar_s[n] * h_{tj-1}[n]   <=   2^-MSS_REPLAY_DECAY_BITS |h_{tj-1}[n]|
 * per state n, where tj is the step its replay started from, and an output
 * y_t lacks sum_n C_t[n] times that (times SiLU(z_t)).  So the difference
 * from the sequential recurrence is bounded by 2^-MSS_REPLAY_DECAY_BITS
 * times the magnitude of the state at the replay start: only a state far
 * above the scale of the outputs shortly before a segment start could make
 * it visible.  Segment lengths depend on the shape (and flags) alone, never
 * on the device or the environment: mss_time_split reports them, and the
 * output bits are a function of the inputs and the shape.
 * MSS_FLAG_EXACT turns the split off: each channel tile scans its whole
 * sequence in one wave, so there is no replay and the result is the plain
 * recurrence in fp32, at the cost of parallelism (B * ceil(D/64) waves for
 * the scans, B * ceil(D/32) for the scan backward, B * H workgroups for the
 * SSD scan). */
#define MSS_REPLAY_DECAY_BITS 24
#define MSS_FLAG_EXACT 1
/* MSS_FLAG_CKPT8: state checkpoints every 8 steps, for the backward pass.
 * Forward calls: h_cache is (B, ceil(L/8), D, N) and holds the state entering
 * steps 0, 8, 16, ... (entry k = h_{8k-1}; entry 0 = h0, or 0) instead of
 * every step's state -- 8 bytes per (m, d) instead of 64.
 * mss_selective_scan_backward: the flag says that h_ckpt carries those
 * checkpoints (from a forward call with the same inputs); the backward then
 * starts every 8-step block from them instead of rebuilding the states, and
 * needs no checkpoint workspace (mss_workspace_bytes with the flag set
 * reports the smaller size).  Without the flag h_ckpt must be NULL. */
#define MSS_FLAG_CKPT8 2
typedef struct mss_dims {
    int32_t struct_size;
    int32_t flags;          /* 0, or MSS_FLAG_EXACT (any other bit: MSS_EINVAL) */
    int64_t batch;          /* B */
    int64_t seq_len;        /* L (ignored by mss_selective_step) */
    int64_t d_inner;        /* D */
    int64_t d_state;        /* N, 1..16 */
    int64_t d_conv;         /* K, 1..8 (ignored by mss_selective_scan) */
} mss_dims;

/* Discretisation of the input term (the caller must choose; no default).
 *   MSS_DISC_ZOH:   bBar = ((exp(dv*A) - 1) / A) * B, as the pages' scan
 *                   computes it (mamba1CpuForward step 8; its backward pass
 *                   differentiates the same form).
 *   MSS_DISC_EULER: bBar = dv * B (the simplified form). */
#define MSS_DISC_ZOH 0
#define MSS_DISC_EULER 1

/* Steps 4 + 5: u = SiLU(b_conv[d] + sum_{k<K, k<=t} w_conv[d*K + k] * x[b, t-k, d]).
 * Tap k = 0 multiplies the current step; there is no contribution from
 * before t = 0 of each batch row, and none across batch rows.
 *   x      (M, D)  in
 *   w_conv (D, K)  in
 *   b_conv (D)     in, may be NULL (= 0)
 *   u      (M, D)  out                                                      */
int mss_conv1d_silu(const mss_dims* dims, const float* x, const float* w_conv,
                    const float* b_conv, float* u, hipStream_t stream);

/* Steps 8 + 9 on a given u:
 *   dv = softplus(delta) = max(delta, 0) + log1p(exp(-|delta|))
 *   A[d,n] = -exp(clamp(A_log[d,n], -10, 5)),  aBar = exp(dv * A)
 *   h_t = aBar * h_{t-1} + bBar(disc) * u_t      (h_{-1} = h0, or 0)
 *   y_t = (D_vec[d] * u_t + sum_n C[r,n] * h_t[n]) * SiLU(z_t)
 *   u, delta, z, y (M, D);  A_log (D, N);  B, C (M, N);  D_vec (D);
 *   h0, h_last (B, D, N);  h_cache (B, L, D, N) = h_t after the update of step t.
 *   Optional (NULL allowed): D_vec (= 0), z (ungated output), h0 (= 0),
 *   h_cache, h_last.  Required: u, delta, A_log, B, C, y.
 *   Time is split into segments processed in parallel (see "Time split"
 *   above for what that drops, and MSS_FLAG_EXACT for the path without it);
 *   the result is otherwise the plain recurrence in fp32.                  */
int mss_selective_scan(const mss_dims* dims, int disc, const float* u, const float* delta,
                       const float* A_log, const float* B, const float* C, const float* D_vec,
                       const float* z, const float* h0, float* y, float* h_cache,
                       float* h_last, hipStream_t stream);

/* Steps 4, 5, 8 and 9 fused into one kernel: mss_conv1d_silu followed by
 * mss_selective_scan, without materialising u.  Same arguments and layouts;
 * x (M, D), w_conv (D, K), b_conv (D, may be NULL) replace u.             */
int mss_mamba1_core(const mss_dims* dims, int disc, const float* x, const float* w_conv,
                    const float* b_conv, const float* delta, const float* A_log,
                    const float* B, const float* C, const float* D_vec, const float* z,
                    const float* h0, float* y, float* h_cache, float* h_last,
                    hipStream_t stream);

/* Row strides (in elements) of the activation-shaped tensors, for reading
 * them in place as column slices of wider buffers: x and z as the two halves
 * of the (M, 2D) input-projection output, delta / B / C as column ranges of
 * the (M, R+2N) x-projection output.  The pages split these with a strided
 * column gather (COL_SLICE_WGSL / dispatchColumnSlice, which replaced a
 * prefix copy that was wrong for more than one row; builderforce-memory-engine
 * 2026.7.14 -> 2026.9.28, src/model/mamba1_block.ts); the strided entry
 * points make that gather unnecessary.
 * Row r of tensor T starts at T + r * T_stride.  Each stride must be at least
 * the row width (D for x, z, delta, y; N for B, C).  In the strided entry
 * points x (or u), z, delta, B, C and y need only 4-byte alignment; the
 * remaining tensors keep the 16-byte rule. */
typedef struct mss_strides {
    int32_t struct_size;    /* sizeof(mss_strides) */
    int32_t reserved;       /* must be 0 */
    int64_t x;              /* x (core) or u (scan) */
    int64_t z;
    int64_t delta;
    int64_t B;
    int64_t C;
    int64_t y;
} mss_strides;

/* mss_selective_scan with row strides; same semantics otherwise. */
int mss_selective_scan_strided(const mss_dims* dims, const mss_strides* strides, int disc,
                               const float* u, const float* delta, const float* A_log,
                               const float* B, const float* C, const float* D_vec,
                               const float* z, const float* h0, float* y, float* h_cache,
                               float* h_last, hipStream_t stream);

/* mss_mamba1_core with row strides; same semantics otherwise. */
int mss_mamba1_core_strided(const mss_dims* dims, const mss_strides* strides, int disc,
                            const float* x, const float* w_conv, const float* b_conv,
                            const float* delta, const float* A_log, const float* B,
                            const float* C, const float* D_vec, const float* z,
                            const float* h0, float* y, float* h_cache, float* h_last,
                            hipStream_t stream);

/* One single-token recurrent step (decode) with carried state; the plainest
 * reading of steps 4-9 for L = 1 with the conv window and h carried over.
 *   x, z, delta, y (B, D);  B, C (B, N);  A_log (D, N);  D_vec (D);
 *   w_conv (D, K);  b_conv (D);
 *   conv_state (B, K-1, D) in/out: the K-1 previous inputs, oldest first;
 *     tap k >= 1 multiplies conv_state[K-1-k]; afterwards the window is
 *     shifted by one and x appended.  May be NULL only when K == 1.
 *   h (B, D, N) in/out: the scan state, updated in place.
 *   Optional: D_vec, z, b_conv (NULL = 0 / ungated / 0).              */
int mss_selective_step(const mss_dims* dims, int disc, const float* x, const float* z,
                       const float* delta, const float* A_log, const float* B, const float* C,
                       const float* D_vec, const float* w_conv, const float* b_conv,
                       float* conv_state, float* h, float* y, hipStream_t stream);

/* ---- Backward passes ------------------------------------------------------
 * The reverse-time adjoint of the pages' CPU mirror (same diff and file,
 * function mamba1CpuBackward: its gate, reverse-time selective-scan, A_log
 * clamp mask, softplus, SiLU and depthwise conv1d parts).
 * Gradients are written, not accumulated.  Both entry points take a caller
 * workspace of at least mss_workspace_bytes bytes for the same dims and
 * device (256-byte aligned, overlapping nothing else; MSS_EWORKSPACE if
 * missing or too small); its contents on entry do not matter and it may be
 * reused once the call's work on `stream` has finished.  Results are
 * deterministic: every sum runs in a fixed order, no atomics.            */

#define MSS_OP_SELECTIVE_SCAN_BACKWARD 1
#define MSS_OP_CONV1D_SILU_BACKWARD 2

/* Workspace size in bytes for `op` (one of MSS_OP_*) on the current device;
 * 0 for empty problems. */
int mss_workspace_bytes(const mss_dims* dims, int op, size_t* bytes);

/* Gradients of the selective scan + gate (the forward of mss_selective_scan,
 * same inputs and layouts) against dout (M, D), the gradient of y:
 *   dY = dout * SiLU(z) (dout when z is NULL), with h the forward states and
 *   g the adjoint carried from step t+1, dh = C[r,:] dY + g:
 *   du (M, D)      = D_vec dY + sum_n dh bBar      (through the scan only:
 *                    the caller adds what u receives elsewhere)
 *   ddelta (M, D)  = sigmoid(delta) sum_n (dh h_{t-1} A aBar + dh u dbBar/ddv)
 *   dA_log (D, N)  = A sum_{b,t} (dh h_{t-1} dv aBar + dh u dbBar/dA),
 *                    0 where A_log <= -10 or A_log >= 5 (outside the clamp)
 *   dB, dC (M, N)  = sum_d dh u dbBar/dB,  sum_d dY h_t
 *   dD_vec (D)     = sum_{b,t} dY u                 (NULL: not computed)
 *   dz (M, D)      = dout y SiLU'(z), y ungated     (required iff z given)
 *   dh0 (B, D, N)  = the adjoint after step 0       (NULL: not computed)
 * Time segments are processed in parallel as in the forward: each rebuilds
 * the forward state entering it and the adjoint leaving it by replays whose
 * starting point has decayed by 2^-MSS_REPLAY_DECAY_BITS (see "Time split";
 * for the adjoint the window runs forward in time from the segment end).
 * MSS_FLAG_EXACT: no split, no replay.                                      */
/* h_ckpt (B, ceil(L/8), D, N): the forward's states entering every 8th step
 * (MSS_FLAG_CKPT8 in dims->flags; NULL otherwise).                        */
int mss_selective_scan_backward(const mss_dims* dims, int disc, const float* u,
                                const float* delta, const float* A_log, const float* B,
                                const float* C, const float* D_vec, const float* z,
                                const float* h0, const float* h_ckpt, const float* dout,
                                float* du, float* ddelta, float* dA_log, float* dB, float* dC,
                                float* dD_vec, float* dz, float* dh0, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc:
 * mss_selective_scan_backward with the workspace taken from a static device
 * array inside the library instead of from the caller.  Same arguments and
 * results (the same kernels), minus the workspace.
 *   - The array holds MSS_NOALLOC_SCRATCH_BYTES (256 MiB) on every GPU the
 *     library runs on, from the time its code is loaded until the process
 *     ends.  A problem whose mss_workspace_bytes(MSS_OP_SELECTIVE_SCAN_BACKWARD)
 *     exceeds it is refused with MSS_ESCRATCH before anything is launched
 *     (B2 L512 D256 needs 3.3 MiB, B4 L2048 D1024 101 MiB, B8 L2048 D1536
 *     294 MiB: refused).  With the forward's checkpoints (MSS_FLAG_CKPT8)
 *     the backward needs no checkpoint workspace: B8 L2048 D1536 then needs
 *     102 MiB.
 *   - The call allocates nothing: no hipMalloc, no hipFree, no allocating
 *     library routine.  Its first call on a device looks up the array's
 *     device address (hipGetSymbolAddress, with that device current).
 *   - All calls on one GPU share the one array, which keeps the last call's
 *     contents (nothing in it needs to start at zero).  Calls that overlap
 *     in time on one GPU -- on two streams, or from two threads -- race on
 *     it: order them on one stream or use the workspace entry point.      */
#define MSS_NOALLOC_SCRATCH_BYTES (256ull << 20)
int mss_selective_scan_backward_noalloc(const mss_dims* dims, int disc, const float* u,
                                        const float* delta, const float* A_log, const float* B,
                                        const float* C, const float* D_vec, const float* z,
                                        const float* h0, const float* h_ckpt, const float* dout,
                                        float* du, float* ddelta, float* dA_log, float* dB,
                                        float* dC, float* dD_vec, float* dz, float* dh0,
                                        hipStream_t stream);

/* Gradients of u = SiLU(conv1d(x)) (mss_conv1d_silu) against du (M, D), the
 * total gradient reaching u:  dc = du * SiLU'(c),
 *   dx (M, D)         = sum_{k, t+k<L} dc[t+k] w_conv[d,k]
 *   dw_conv (D, K)    = sum_{b, t>=k} dc[t] x[t-k]
 *   db_conv (D)       = sum_{b,t} dc[t]            (NULL: not computed)   */
int mss_conv1d_silu_backward(const mss_dims* dims, const float* x, const float* w_conv,
                             const float* b_conv, const float* du, float* dx, float* dw_conv,
                             float* db_conv, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ---- Mamba-2 SSD scan --------------------------------------------------------
 * The recurrence that the pages' Mamba2Block dispatches as ssd_chunk_forward
 * (diff 2026.7.14 -> 2026.9.28, src/model/mamba2_block.ts: x (M, D = H*P),
 * dt (M, H), B and C (M, G*N) split from the projections).  The pages do not
 * show its arithmetic; this is the plainest reading consistent with the
 * Mamba-1 path: per batch row and head h of group g = h / (H/G),
 *   dv = softplus(dt[r, h] + dt_bias[h]),  A_h = -exp(clamp(A_log[h], -10, 5))
 *   S_h[p, n] <- exp(dv A_h) S_h[p, n] + f x[r, h*P + p] B[r, g*N + n]
 *   y[r, h*P + p] = sum_n C[r, g*N + n] S_h[p, n] + D_vec[h] x[r, h*P + p]
 * with f = dv (MSS_DISC_EULER, the Mamba-2 form) or expm1(dv A_h) / A_h
 * (MSS_DISC_ZOH, the discretisation of the pages' Mamba-1 path).
 * Computed in chunks on the matrix cores (fp32 MFMA); time segments are
 * processed in parallel, each rebuilding its initial state by a replay whose
 * start has decayed by 2^-MSS_REPLAY_DECAY_BITS (see "Time split"; here the
 * decay is the head's scalar exp(A_h sum dv)).  MSS_FLAG_EXACT: no split. */
typedef struct mss_ssd_dims {
    int32_t struct_size;    /* sizeof(mss_ssd_dims) */
    int32_t flags;          /* 0, or MSS_FLAG_EXACT (any other bit: MSS_EINVAL) */
    int64_t batch;          /* B */
    int64_t seq_len;        /* L */
    int64_t n_heads;        /* H */
    int64_t head_dim;       /* P: 16, 32, 64 or 128 */
    int64_t d_state;        /* N: 16, 32, 64 or 128 */
    int64_t n_groups;       /* G: divides H */
} mss_ssd_dims;

/*   x, y (M, H*P);  dt (M, H);  A_log (H);  B, C (M, G*N);
 *   D_vec, dt_bias (H), may be NULL (= 0);
 *   h0, h_last (B, H, P, N), may be NULL (h0 = 0 / not written).
 * A sequence of length 0 still defines h_last (= h0, or zeros).          */
int mss_ssd_scan(const mss_ssd_dims* dims, int disc, const float* x, const float* dt, const float* A_log,
                 const float* B, const float* C, const float* D_vec, const float* dt_bias,
                 const float* h0, float* y, float* h_last, hipStream_t stream);

/* ---- Time split ----------------------------------------------------------
 * The segment length, in steps, that a call with these dims (flags
 * included) uses, for callers and tests that need to know where segments
 * start.  op: MSS_OP_SELECTIVE_SCAN (mss_selective_scan, mss_mamba1_core and
 * their strided forms) or MSS_OP_SELECTIVE_SCAN_BACKWARD.  The scans cut the
 * flattened (tile, t) space, tile = b * ceil(D/T) + d / T with T = 64
 * channels (forward) or 32 (backward) and t running fastest, into pieces of
 * *segment_steps steps (a multiple of 8); a segment starts wherever
 * (tile * Lp + t) is a multiple of *segment_steps, with Lp = L rounded up to
 * a multiple of 8 (so segments start at multiples of 8).  0 for empty
 * problems.                                                                 */
#define MSS_OP_SELECTIVE_SCAN 3
int mss_time_split(const mss_dims* dims, int op, int64_t* segment_steps);

/* The same for mss_ssd_scan: every (batch row, head) sequence is cut into
 * segments of *segment_steps steps starting at t = 0.                       */
int mss_ssd_time_split(const mss_ssd_dims* dims, int64_t* segment_steps);

/* Human-readable text for a status code (static storage). */
const char* mss_strerror(int status);

/* MSS_VERSION of the library that was loaded. */
int mss_version(void);

/* The hipError_t of the last MSS_EHIP returned on the calling thread. */
int mss_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MSS_H */
