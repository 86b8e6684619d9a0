"""Throughput of the Mamba-1 block core on one MI355X.

One step = one pass of the whole hot path over one batch: causal depthwise
conv1d + SiLU, softplus(delta), clamped A, discretisation, selective scan,
y = sum_n C h + D u, SiLU(z) gate -- the fused mss_mamba1_core kernel -- on the
4 x 8192 x 5120 (d_state 16, d_conv 4) workload of a 2.8B-class Mamba-1
block, inputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--disc zoh|euler] [--no-cpu-baseline]

Order of work: the side measurements on the GPU (the other workloads, the
other discretisation, backward, SSD, decode) run first, then about 100 ms of
the step, W warm-up steps and the K timed steps, then everything that times
the CPU oracle.  The part's clock ramps up over the first ~20 ms of sustained
load (a cold SSD call measures 1.3-1.4 ms, the twentieth 1.07 ms), so every
timing here, side measurements included, follows about 100 ms of the same
work: the figures are those of a continuously loaded GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                      # MI355X HBM3E, AMD published
METRIC = "selective-scan M·D elements/s and achieved HBM GB/s (% of peak), 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_mamba1_core_b4_l8192_d5120.txt")
COPY_BYTES = 1 << 30                      # calibration copy: 1 GiB read + 1 GiB written
WARM_MS = 100.0                           # sustained load before each side timing (see _settle)
KERNEL_SOURCES = ("scan_kernel.hip", "device_math.h", "launch.h")


def kernel_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mamba_selective_scan_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w) -> int:
    """Bytes the fused kernel must move: x, delta, z in and y out per (m, d);
    B and C per (m, n); the per-channel parameters once."""
    M, D, N, K = w.M, w.d_inner, w.d_state, w.d_conv
    return 4 * (4 * M * D + 2 * M * N + D * N + D * (K + 2))


# Secondary roofline, VALU issue.  Non-packed fp32 issue: 256 CUs x 4 SIMDs x
# 16 lanes per cycle x 2.4 GHz = 39.3e12 lane operations per second, where an
# FMA, multiply or add takes one issue slot and a transcendental (exp, log,
# rcp) two (measured: v_exp_f32 runs at half the FMA rate).  The published
# 157.3 TFLOP/s fp32 vector peak counts packed FMAs (two per lane per cycle,
# two flops each), a form this library does not use; the flops against it
# are reported beside.
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
FP32_VECTOR_PEAK_TFLOPS = 157.3


def algorithmic_ops(w, disc) -> int:
    """fp32 operations the fused kernel's formulas need per launch.  Per
    (m, d, n): dv*A, exp, then ZOH u/A*B (two multiplies), h + K and the
    update FMA, or EULER (dv u)*B and the update FMA, and the y FMA: 7 (ZOH)
    or 5 (EULER).  Per (m, d): the K conv FMAs, SiLU of the conv (5), softplus
    (8), the SiLU gate and its product (6), the skip (1), EULER's dv*u (1)."""
    M, D, N, K = w.M, w.d_inner, w.d_state, w.d_conv
    per_state = 7 if disc == "zoh" else 5
    per_md = K + 5 + 8 + 6 + 1 + (0 if disc == "zoh" else 1)
    return M * D * (N * per_state + per_md)


def algorithmic_issue(w, disc):
    """(issue slots, transcendentals, flops) per launch of the fused kernel:
    the operations of algorithmic_ops with each transcendental taking a
    second slot (per (m, d, n) one exp; per (m, d) two each in SiLU of the
    conv, softplus and the gate), and flops with an FMA as two."""
    M, D, N, K = w.M, w.d_inner, w.d_state, w.d_conv
    ops = algorithmic_ops(w, disc)
    trans = M * D * (N + 6)
    # per (m, d, n): ZOH mul, exp, 2 mul, add, 2 FMA = 9 flops; EULER 7
    per_state = 9 if disc == "zoh" else 7
    per_md = 2 * K + 5 + 8 + 6 + 2 + (0 if disc == "zoh" else 1)
    return ops + trans, trans, M * D * (N * per_state + per_md)


def roofline(w, disc, kern_ms, traffic, digest):
    """HBM roofline of the fused kernel (the metric's), with VALU issue beside."""
    abytes = algorithmic_bytes(w)
    achieved = abytes / (kern_ms / 1e3) / 1e9
    issue, trans, flops = algorithmic_issue(w, disc)
    ops = algorithmic_ops(w, disc)
    t = kern_ms / 1e3
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "algorithmic_bytes": abytes, "kernel_ms": kern_ms, "kernel_digest": digest,
            "alu": {"note": "secondary: the kernel is VALU-issue bound; peak = non-packed "
                            "fp32 issue 256 CU x 4 SIMD x 16 lanes x 2.4 GHz, transcendentals "
                            "at two slots",
                    "algorithmic_ops": ops, "issue_slots": issue, "transcendentals": trans,
                    "achieved_issue_T_per_s": issue / t / 1e12, "peak_T_per_s": ALU_PEAK_TOPS,
                    "issue_frac": issue / t / 1e12 / ALU_PEAK_TOPS,
                    "flops": flops, "achieved_TFLOPs": flops / t / 1e12,
                    "published_fp32_vector_peak_TFLOPs": FP32_VECTOR_PEAK_TFLOPS,
                    "frac_of_published_fp32_peak": flops / t / 1e12 / FP32_VECTOR_PEAK_TFLOPS}}


def measured_traffic(digest: str):
    """HBM bytes per launch of the fused kernel from rocprofv3 FETCH_SIZE and
    WRITE_SIZE counters (calibrated on a plain copy), read from the committed
    summary, if it was taken on this exact kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith(" "))
    except OSError:
        return None
    if kv.get("kernel_digest", "").strip() != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def copy_calibration(reps: int):
    """A plain device copy of COPY_BYTES, for calibrating HBM byte counters."""
    import torch
    src = torch.ones(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": reps}), flush=True)


def _settle(fn, stream, warm, warm_ms):
    """fn() at least `warm` times and until about `warm_ms` of GPU time has
    passed: the part's clock ramps up over the first ~20 ms of sustained
    load (an SSD call measures 1.3-1.4 ms at first, 1.07 ms from about the
    twentieth), so a timing taken right after host-side work would measure
    the ramp."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, spent = max(warm, 1), 0.0
    while True:
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        el = a.elapsed_time(b)
        spent += el
        if spent >= warm_ms:
            return
        per = max(el / n, 1e-3)
        n = min(2000, int((warm_ms - spent) / per) + 1)


def _time_ms(fn, stream, reps, warm=2, warm_ms=WARM_MS):
    """Mean hipEvent time of fn() on `stream`, in ms, after _settle."""
    import torch
    _settle(fn, stream, warm, warm_ms)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _event_times(fn, stream, reps, before=None):
    """Per-call hipEvent times of fn() on `stream` (ms); before() runs ahead
    of each call, outside the timed interval."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        if before is not None:
            before()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _stats(ts):
    return {"mean": float(np.mean(ts)), "median": float(np.median(ts)), "min": float(np.min(ts)),
            "calls": len(ts)}


def extras(w, inp, d, y, disc, stream):
    """Side measurements: the other discretisation, the fused core reading
    column slices of the projection outputs, the unfused path (conv kernel,
    then the scan on u), and the decode workload (256 sequences x 5120
    channels, 64 consecutive single-token steps)."""
    import torch
    import mamba_selective_scan_causal_amd as mss
    from mamba_selective_scan_causal_amd import inputs as gen
    res = {}
    other = "euler" if disc == "zoh" else "zoh"
    kw = dict(batch=w.batch, seq_len=w.seq_len, out=y, stream=stream)
    t = _time_ms(lambda: mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"],
                                         d["B"], d["C"], d["D_vec"], d["z"], None, disc=other,
                                         **kw), stream, 10)
    res[f"fused_{other}_ms"] = t
    # a plain 1 GiB device copy (read + write) for scale: the HBM rate a
    # simple streaming kernel reaches on this part
    src = torch.ones(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    tcopy = _time_ms(lambda: dst.copy_(src), stream, 10)
    res["copy_1GiB"] = {"ms": tcopy, "GBps": 2 * COPY_BYTES / tcopy / 1e6,
                        "frac_of_peak": 2 * COPY_BYTES / tcopy / 1e6 / HBM_PEAK_GBS}
    del src, dst
    # cold: a 512 MB buffer is written between calls, so that the inputs are
    # not served from the 256 MB last-level cache
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    cold = _event_times(lambda: mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"],
                                                d["A_log"], d["B"], d["C"], d["D_vec"], d["z"],
                                                None, disc=disc, **kw),
                        stream, 10, before=lambda: flush.fill_(1.0))
    res["fused_cold_ms"] = _stats(cold)
    # with the per-step state cache (a9): 64 more bytes written per (m, d)
    hc = torch.empty((w.batch, w.seq_len, w.d_inner, w.d_state), device="cuda")
    thc = _time_ms(lambda: mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"],
                                           d["A_log"], d["B"], d["C"], d["D_vec"], d["z"], None,
                                           disc=disc, h_cache=hc, **kw), stream, 5)
    hc_bytes = algorithmic_bytes(w) + 4 * w.M * w.d_inner * w.d_state
    res["fused_hcache"] = {"ms": thc, "algorithmic_bytes": hc_bytes,
                           "GBps": hc_bytes / thc / 1e6,
                           "frac_of_peak": hc_bytes / thc / 1e6 / HBM_PEAK_GBS}
    del hc
    # the layout inside a Mamba-1 block: x and z the two halves of the
    # (M, 2D) in_proj output, B and C columns of the (M, R + 2N) x_proj
    # output (R = D / 16, the dt rank), read in place through row strides
    Dm, Nm = w.d_inner, w.d_state
    R = Dm // 16
    XZ = torch.empty((w.M, 2 * Dm), device="cuda")
    XZ[:, :Dm].copy_(d["x"])
    XZ[:, Dm:].copy_(d["z"])
    XP = torch.zeros((w.M, R + 2 * Nm), device="cuda")
    XP[:, R:R + Nm].copy_(d["B"])
    XP[:, R + Nm:].copy_(d["C"])

    def strided(m):
        return lambda: mss.mamba1_core(XZ[:, :Dm], d["w_conv"], d["b_conv"], d["delta"],
                                       d["A_log"], XP[:, R:R + Nm], XP[:, R + Nm:], d["D_vec"],
                                       XZ[:, Dm:], None, disc=m, **kw)

    def dense(m):
        return lambda: mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"],
                                       d["B"], d["C"], d["D_vec"], d["z"], None, disc=m, **kw)
    # alternating rounds, so that both layouts see the same clock
    ts = {k: [] for k in ("s", "d")}
    _settle(dense(disc), stream, 2, WARM_MS)
    for _ in range(4):
        ts["s"] += _event_times(strided(disc), stream, 5)
        ts["d"] += _event_times(dense(disc), stream, 5)
    res["fused_strided"] = {"layout": f"x, z halves of ({w.M}, {2 * Dm}); B, C columns of "
                                      f"({w.M}, {R + 2 * Nm}); delta, y dense",
                            "disc": disc,
                            "strided_ms": _stats(ts["s"]), "dense_ms": _stats(ts["d"])}
    del XZ, XP
    u = torch.empty_like(d["x"])
    tc = _time_ms(lambda: mss.conv1d_silu(d["x"], d["w_conv"], d["b_conv"], batch=w.batch,
                                          seq_len=w.seq_len, out=u, stream=stream), stream, 10)
    ts = {m: _time_ms(lambda: mss.selective_scan(u, d["delta"], d["A_log"], d["B"], d["C"],
                                                 d["D_vec"], d["z"], None, disc=m, **kw),
                      stream, 10)
          for m in (disc, other)}
    MD = w.M * w.d_inner
    res["unfused"] = {"conv1d_silu_ms": tc, "conv1d_silu_GBps": 8 * MD / tc / 1e6,
                      "scan_on_u_ms": ts[disc], f"scan_on_u_{other}_ms": ts[other],
                      "total_ms": tc + ts[disc]}
    del u
    del flush
    res["decode"] = decode_extras(disc, stream)
    res["backward"] = backward_extras(w, d, stream, with_oracle=False)
    res["ssd"] = ssd_extras(stream, reps=10, with_oracle=False)
    res["workloads"] = workloads_extras(stream)
    return res


def oracle_extras(w, inp, disc, extra):
    """The CPU oracle's rates for the side measurements, after the GPU work."""
    extra["cpu_oracle_1core"] = cpu_baseline(w, inp, disc, target_s=4.0, threads=1)
    extra["backward"]["cpu_oracle"] = backward_oracle_rate(w)
    from mamba_selective_scan_causal_amd import inputs as gen
    sw = gen.SSD_2P7B
    extra["ssd"]["cpu_oracle"] = ssd_oracle_rate(sw, gen.generate_ssd(sw))
    for name, r in workloads_oracle().items():
        extra["workloads"][name]["cpu_oracle_1core"] = r


def workload_bytes(w, h_cache: bool) -> int:
    """Algorithmic bytes of a fused call: algorithmic_bytes, plus the state
    cache (4 N bytes per (m, d)) when it is written."""
    return algorithmic_bytes(w) + (4 * w.M * w.d_inner * w.d_state if h_cache else 0)


def workloads_extras(stream, reps=50):
    """The fused core on the other sequence workloads (1 x 64 x 32 with the
    clamp path, 2 x 512 x 256 and 8 x 2048 x 1536): both discretisations,
    with the state cache where the workload emits it; median of `reps`
    event-timed calls after a warm-up."""
    import torch
    import mamba_selective_scan_causal_amd as mss
    from mamba_selective_scan_causal_amd import inputs as gen
    out = {}
    for w in (gen.TINY_CLAMP, gen.SMALL, gen.MAMBA_130M):
        inp = gen.generate(w)
        d = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
        y = torch.empty((w.M, w.d_inner), device="cuda")
        hc = (torch.empty((w.batch, w.seq_len, w.d_inner, w.d_state), device="cuda")
              if w.hcache else False)
        res = {"h_cache": w.hcache}
        for disc in ("zoh", "euler"):
            def f(disc=disc):
                mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"],
                                d["B"], d["C"], d["D_vec"], d["z"], None, batch=w.batch,
                                seq_len=w.seq_len, disc=disc, out=y, h_cache=hc, stream=stream)
            _settle(f, stream, 2, WARM_MS)
            ts = _event_times(f, stream, reps)
            ms = float(np.median(ts))
            nb = workload_bytes(w, w.hcache)
            res[disc] = {"ms": ms, "min_ms": float(np.min(ts)),
                         "elements_per_s": w.M * w.d_inner / (ms / 1e3),
                         "algorithmic_bytes": nb, "GBps": nb / ms / 1e6,
                         "frac_of_hbm_peak": nb / ms / 1e6 / HBM_PEAK_GBS}
        out[w.name] = res
        del d, y, hc
    return out


def workloads_oracle(target_s=3.0):
    """The oracle as it stands on one core on the same workloads (whole
    workload for the two small ones, a bounded sample of whole columns of
    the 8 x 2048 x 1536 one), ZOH."""
    from mamba_selective_scan_causal_amd import inputs as gen
    out = {}
    for w in (gen.TINY_CLAMP, gen.SMALL, gen.MAMBA_130M):
        inp = gen.generate(w)
        out[w.name] = cpu_baseline(w, inp, "zoh", target_s=target_s, threads=1)
    return out


def decode_extras(disc, stream):
    """The decode workload (256 sequences x 5120 channels, d_state 16): 64
    consecutive single-token steps with the state carried in place, the
    same 64 steps replayed from a captured HIP graph, and 16 single steps
    each after a 512 MB write (cold last-level cache)."""
    import torch
    import mamba_selective_scan_causal_amd as mss
    from mamba_selective_scan_causal_amd import inputs as gen
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    dw = gen.DECODE
    dinp = gen.generate(dw)
    dd = {k: torch.from_numpy(v).cuda() for k, v in dinp.items()}
    yd = torch.empty((dw.batch, dw.d_inner), device="cuda")

    def decode64():
        for s_ in range(dw.seq_len):
            mss.selective_step(dd["x"][s_], dd["z"][s_], dd["delta"][s_], dd["A_log"],
                               dd["B"][s_], dd["C"][s_], dd["D_vec"], dd["w_conv"],
                               dd["b_conv"], dd["conv_state"], dd["h"], disc=disc, out=yd,
                               stream=stream)

    t64 = _time_ms(decode64, stream, 3, warm=1)

    # the same 64 steps captured once as a HIP graph and replayed
    def decode64_current():
        for s_ in range(dw.seq_len):
            mss.selective_step(dd["x"][s_], dd["z"][s_], dd["delta"][s_], dd["A_log"],
                               dd["B"][s_], dd["C"][s_], dd["D_vec"], dd["w_conv"],
                               dd["b_conv"], dd["conv_state"], dd["h"], disc=disc, out=yd)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode64_current()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode64_current()
    t64g = _time_ms(graph.replay, torch.cuda.current_stream(), 3, warm=1)
    del graph

    def one_step():
        mss.selective_step(dd["x"][0], dd["z"][0], dd["delta"][0], dd["A_log"], dd["B"][0],
                           dd["C"][0], dd["D_vec"], dd["w_conv"], dd["b_conv"],
                           dd["conv_state"], dd["h"], disc=disc, out=yd, stream=stream)

    step_cold = _event_times(one_step, stream, 16, before=lambda: flush.fill_(1.0))
    BD, N, K = dw.batch * dw.d_inner, dw.d_state, dw.d_conv
    step_bytes = BD * (16 + 8 * N + 8 * (K - 1)) + dw.batch * N * 8 + dw.d_inner * (N + K + 2) * 4
    return {"workload": dw.name, "steps": dw.seq_len, "us_per_step": t64 * 1e3 / dw.seq_len,
            "algorithmic_bytes_per_step": step_bytes,
            "GBps": step_bytes / (t64 / dw.seq_len) / 1e6,
            "note": "h + conv window (~100 MB) fit the 256 MB last-level cache",
            "graph_us_per_step": t64g * 1e3 / dw.seq_len,
            "cold_us_per_step": _stats([t * 1e3 for t in step_cold]),
            "cold_GBps": step_bytes / float(np.median(step_cold)) / 1e6}


def backward_extras(w, d, stream, reps=5, with_oracle=True):
    """The backward passes on the same workload (ZOH), as training runs them:
    the forward (the scan on u = SiLU(conv(x))) writes its 8-step state
    checkpoints, the scan backward starts from them (main kernel + fixed-
    order reduction kernel; seeded N(0, 1) output gradient); then the
    conv1d + SiLU backward.  The scan backward without checkpoints (it then
    rebuilds the forward states itself) is timed beside."""
    import torch
    import mamba_selective_scan_causal_amd as mss
    from mamba_selective_scan_causal_amd import inputs as gen
    M, D, N = w.M, w.d_inner, w.d_state
    u = mss.conv1d_silu(d["x"], d["w_conv"], d["b_conv"], batch=w.batch, seq_len=w.seq_len,
                        stream=stream)
    dout = torch.from_numpy(gen.cotangent(w)).cuda()
    kw = dict(batch=w.batch, seq_len=w.seq_len, stream=stream)
    y = torch.empty((M, D), device="cuda")
    ck = torch.empty((w.batch, mss.ckpt_steps(w.seq_len), D, N), device="cuda")

    def fwd_ck():
        mss.selective_scan(u, d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"], d["z"], None,
                           disc="zoh", out=y, h_cache=ck, ckpt8=True, **kw)
    t_fwd_ck = _time_ms(fwd_ck, stream, reps)
    t_core_ck = _time_ms(lambda: mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"],
                                                 d["A_log"], d["B"], d["C"], d["D_vec"], d["z"],
                                                 None, disc="zoh", out=y, h_cache=ck,
                                                 ckpt8=True, **kw), stream, reps)
    nb = mss.workspace_bytes(mss.OP_SELECTIVE_SCAN_BACKWARD, batch=w.batch, seq_len=w.seq_len,
                             d_inner=D, d_state=N)
    nb_ck = mss.workspace_bytes(mss.OP_SELECTIVE_SCAN_BACKWARD, batch=w.batch,
                                seq_len=w.seq_len, d_inner=D, d_state=N, ckpt8=True)
    ws = torch.empty(nb + 256, dtype=torch.uint8, device="cuda")
    box = {}

    def sb_ck():
        box["g"] = mss.selective_scan_backward(u, d["delta"], d["A_log"], d["B"], d["C"],
                                               d["D_vec"], d["z"], None, dout, disc="zoh",
                                               workspace=ws, h_ckpt=ck, **kw)

    def sb():
        mss.selective_scan_backward(u, d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"],
                                    d["z"], None, dout, disc="zoh", workspace=ws, **kw)
    fwd_ck()
    t_sb = _time_ms(sb_ck, stream, reps)
    t_sb_plain = _time_ms(sb, stream, reps)
    du = box["g"]["du"]
    nc = mss.workspace_bytes(mss.OP_CONV1D_SILU_BACKWARD, batch=w.batch, seq_len=w.seq_len,
                             d_inner=D, d_state=1, d_conv=w.d_conv)
    wsc = torch.empty(nc + 256, dtype=torch.uint8, device="cuda")
    t_cb = _time_ms(lambda: mss.conv1d_silu_backward(d["x"], d["w_conv"], d["b_conv"], du,
                                                     workspace=wsc, **kw), stream, reps)
    # algorithmic bytes: u, delta, z, dout in and du, ddelta, dz out per (m, d);
    # B, C in and dB, dC out per (m, n); x, du in and dx out for the conv
    sb_bytes = 4 * (7 * M * D + 4 * M * N + 3 * D * N + 2 * D)
    cb_bytes = 4 * (3 * M * D + 2 * D * (w.d_conv + 1))
    res = {"disc": "zoh",
           "scan_backward_ms": t_sb,
           "scan_backward_note": "from the forward's 8-step state checkpoints (MSS_FLAG_CKPT8)",
           "workspace_bytes": nb_ck,
           "scan_backward_algorithmic_bytes": sb_bytes,
           "scan_backward_GBps": sb_bytes / t_sb / 1e6,
           "scan_backward_elements_per_s": M * D / (t_sb / 1e3),
           "scan_backward_without_checkpoints_ms": t_sb_plain,
           "workspace_bytes_without_checkpoints": nb,
           "forward_scan_with_checkpoints_ms": t_fwd_ck,
           "fused_core_with_checkpoints_ms": t_core_ck,
           "conv1d_silu_backward_ms": t_cb, "conv1d_silu_backward_GBps": cb_bytes / t_cb / 1e6,
           "total_ms": t_sb + t_cb}
    if with_oracle:
        res["cpu_oracle"] = backward_oracle_rate(w)
    return res


def backward_oracle_rate(w, channels=512):
    """The backward oracle as it stands on a bounded part of the same
    workload: one batch row, the first `channels` channels, all L steps."""
    import oracle
    from mamba_selective_scan_causal_amd import inputs as gen
    cores = len(os.sched_getaffinity(0))
    sub = w.with_(batch=1, d_inner=channels)
    inp = gen.generate(sub)
    u = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=1,
                           seq_len=w.seq_len).astype(np.float32)
    dout = gen.cotangent(sub)
    t0 = time.perf_counter()
    oracle.selective_scan_backward(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                   inp["D_vec"], inp["z"], None, dout, batch=1,
                                   seq_len=w.seq_len, disc="zoh", nthreads=cores)
    t = time.perf_counter() - t0
    el = w.seq_len * channels
    return {"value": el / t, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "sample": f"1 x {w.seq_len} x {channels} (b, t, d) of the same shape, fp64 C, "
                      f"{t:.1f} s"}


MFMA_F32_PEAK_TFLOPS = 157.3          # MI355X dense fp32 matrix, AMD published
SSD_CHUNK = 32


def ssd_flops(w) -> int:
    """Dense work of the chunked SSD form with the causal half of the two
    quadratic terms: per (step, head) Q N / 2 + Q P / 2 multiply-adds for
    (C B^T) and (L o C B^T) X, and N P each for C S and the state update."""
    Q, N, P = SSD_CHUNK, w.d_state, w.head_dim
    return 2 * w.M * w.n_heads * (Q * N // 2 + Q * P // 2 + 2 * N * P)


def ssd_extras(stream, reps=5, with_oracle=True):
    """The Mamba-2 SSD scan (mss_ssd_scan) on B4 L8192 H80 P64 N128 G1."""
    import torch
    import mamba_selective_scan_causal_amd as mss
    from mamba_selective_scan_causal_amd import inputs as gen
    w = gen.SSD_2P7B
    inp = gen.generate_ssd(w)
    d = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    y = torch.empty((w.M, w.n_heads * w.head_dim), device="cuda")
    t = _time_ms(lambda: mss.ssd_scan(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D_vec"],
                                      d["dt_bias"], None, batch=w.batch, seq_len=w.seq_len,
                                      head_dim=w.head_dim, d_state=w.d_state,
                                      n_groups=w.n_groups, disc="euler", out=y,
                                      stream=stream),
                 stream, reps)
    fl = ssd_flops(w)
    bytes_ = 4 * (2 * w.M * w.n_heads * w.head_dim + w.M * w.n_heads
                  + 2 * w.M * w.n_groups * w.d_state)
    tf = fl / t / 1e9
    res = {"workload": w.name, "disc": "euler", "ms": t, "algorithmic_flops": fl, "TFLOPs": tf,
           "frac_of_fp32_mfma_peak": tf / MFMA_F32_PEAK_TFLOPS,
           "algorithmic_bytes": bytes_, "GBps": bytes_ / t / 1e6,
           "tokens_per_s": w.M / (t / 1e3),
           "head_steps_per_s": w.M * w.n_heads / (t / 1e3)}
    if with_oracle:
        res["cpu_oracle"] = ssd_oracle_rate(w, inp)
    return res


def ssd_oracle_rate(w, inp, heads=4):
    """The SSD oracle as it stands on `heads` heads of the same workload (all
    batch rows and steps), on all host cores."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    hs = list(range(heads))
    P = w.head_dim
    cols = np.concatenate([np.arange(h * P, (h + 1) * P) for h in hs])
    t0 = time.perf_counter()
    oracle.ssd_scan(np.ascontiguousarray(inp["x"][:, cols]), np.ascontiguousarray(inp["dt"][:, hs]),
                    inp["A_log"][hs], inp["B"], inp["C"], inp["D_vec"][hs], inp["dt_bias"][hs],
                    None, batch=w.batch, seq_len=w.seq_len, n_heads=heads, head_dim=P,
                    d_state=w.d_state, n_groups=w.n_groups, disc="euler", nthreads=cores)
    t = time.perf_counter() - t0
    return {"value": w.M * heads / t, "unit": "head_steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {w.n_heads} heads, all {w.batch} x {w.seq_len} steps, "
                      f"fp64 C, {t:.1f} s"}


def cpu_baseline(w, inp, disc, target_s=15.0, threads=None):
    """The oracle as it stands, on a bounded sample of whole (b, d) columns of
    the same workload, on all host cores it may use (or on `threads`)."""
    import oracle
    cores = threads or len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    allcols = w.batch * w.d_inner

    def run(ncols):
        cols = np.sort(rng.choice(allcols, size=ncols, replace=False))
        t0 = time.perf_counter()
        oracle.mamba1_core(inp["x"], inp["w_conv"], inp["b_conv"], inp["delta"], inp["A_log"],
                           inp["B"], inp["C"], inp["D_vec"], inp["z"], None, batch=w.batch,
                           seq_len=w.seq_len, disc=disc, cols=cols, nthreads=cores)
        return time.perf_counter() - t0

    n0 = 4 * cores
    t = run(n0)
    ncols = int(min(allcols, max(n0, n0 * target_s / max(t, 1e-3))))
    ncols = max(cores, ncols // cores * cores)
    t = run(ncols)
    el = ncols * w.seq_len
    return {"value": el / t, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "sample": f"{ncols} whole (b,d) columns x {w.seq_len} steps of the same workload "
                      f"({el} of {w.M * w.d_inner} M*D elements), fp64 C, {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--disc", default="zoh", choices=("zoh", "euler"))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the side measurements (other mode, unfused path, decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--part", default="all", choices=("all", "backward", "ssd", "workloads", "decode"),
                    help="backward: only the backward passes on the same workload; ssd: only "
                         "the Mamba-2 SSD scan; workloads: only the fused core on the three "
                         "smaller workloads; decode: only the decode steps (one JSON line of "
                         "timings, for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return

    import torch
    import mamba_selective_scan_causal_amd as mss
    from mamba_selective_scan_causal_amd import inputs as gen

    if args.part == "workloads":
        r = workloads_extras(torch.cuda.current_stream(), reps=max(args.steps, 1))
        if not args.no_cpu_baseline:
            for name, o in workloads_oracle().items():
                r[name]["cpu_oracle_1core"] = o
        print(json.dumps(r))
        return
    if args.part == "decode":
        print(json.dumps(decode_extras(args.disc, torch.cuda.current_stream())))
        return
    w = gen.MAMBA_2P8B
    inp = gen.generate(w)
    d = {k: torch.from_numpy(v).cuda() for k, v in inp.items()}
    if args.part == "ssd":
        print(json.dumps(ssd_extras(torch.cuda.current_stream(), reps=max(args.steps, 1),
                                    with_oracle=not args.no_cpu_baseline)))
        return
    if args.part == "backward":
        res = backward_extras(w, d, torch.cuda.current_stream(), reps=max(args.steps, 1),
                              with_oracle=not args.no_cpu_baseline)
        res["workload"] = w.name
        print(json.dumps(res))
        return
    y = torch.empty((w.M, w.d_inner), device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"], d["B"], d["C"],
                        d["D_vec"], d["z"], None, batch=w.batch, seq_len=w.seq_len,
                        disc=args.disc, out=y, stream=stream)

    extra = None
    if not args.no_extras:
        extra = extras(w, inp, d, y, args.disc, stream)
    # the clock settles on this kernel (about 100 ms of it) before the W
    # warm-up steps; the timed region is exactly K steps
    _settle(step, stream, 1, WARM_MS)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_times = [a.elapsed_time(b) for a, b in ev]
    kern_ms = float(np.mean(kern_times))
    ms_per_step = wall * 1e3 / args.steps
    elems = w.M * w.d_inner
    value = elems / (ms_per_step / 1e3)
    digest = kernel_digest()
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq_len,
                   "d_inner": w.d_inner, "d_state": w.d_state, "d_conv": w.d_conv,
                   "disc": args.disc, "h_cache": False, "kernel": "mss_mamba1_core (fused)"},
        # The metric's roofline: algorithmic HBM bytes over the mean event
        # time of the fused kernel, against 8 TB/s.  The kernel is bound by
        # VALU issue; that fraction is in roofline.alu.
        "roofline": roofline(w, args.disc, kern_ms, measured_traffic(digest), digest),
        "kernel_ms": _stats(kern_times),
    }
    if extra is not None:
        if not args.no_cpu_baseline:
            oracle_extras(w, inp, args.disc, extra)
        out["extra"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.disc)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
