"""Concurrency and graph capture on the GPU.

The library keeps no device state, so calls on different streams may overlap,
and a call captured into a HIP graph (torch.cuda.CUDAGraph, whose capture
stream is the current stream the binding passes down) replays the same
kernels.  Each replay here is preceded by eager work and a synchronisation
and compared bitwise with the eager result: every kernel is deterministic.
Graphs are captured only around calls that enqueue kernels (no memset node:
zeroing inside the library is a fill kernel)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import mamba_selective_scan_causal_amd as mss
from mamba_selective_scan_causal_amd import inputs as gen
from gpu_util import announce, assert_close, dev, host

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(autouse=True)
def _announce(request):
    announce(request.node.nodeid)
    yield


def _core(d, w, disc, y, hl, stream=None):
    mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"], d["B"], d["C"],
                    d["D_vec"], d["z"], d.get("h0"), batch=w.batch, seq_len=w.seq_len,
                    disc=disc, h_last=hl, out=y, stream=stream)


def test_two_streams_overlap():
    """Two fused calls on two streams (different workloads, launched back to
    back without waiting) equal the same calls run one after the other."""
    import torch
    wa = gen.SMALL.with_(name="stream_a", batch=2, seq_len=3000, d_inner=256, h0=True)
    wb = gen.SMALL.with_(name="stream_b", batch=3, seq_len=1700, d_inner=192, seed_index=77)
    da = {k: dev(v) for k, v in gen.generate(wa).items()}
    db = {k: dev(v) for k, v in gen.generate(wb).items()}
    ref = []
    for d, w, disc in ((da, wa, "zoh"), (db, wb, "euler")):
        y = torch.empty((w.M, w.d_inner), device="cuda")
        hl = torch.empty((w.batch, w.d_inner, w.d_state), device="cuda")
        _core(d, w, disc, y, hl)
        torch.cuda.synchronize()
        ref.append((y.clone(), hl.clone()))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for d, w, disc, s in ((da, wa, "zoh", s1), (db, wb, "euler", s2)):
        y = torch.full((w.M, w.d_inner), float("nan"), device="cuda")
        hl = torch.full((w.batch, w.d_inner, w.d_state), float("nan"), device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            _core(d, w, disc, y, hl, stream=s)
        outs.append((y, hl))
    torch.cuda.synchronize()
    for (y, hl), (ry, rhl) in zip(outs, ref):
        assert torch.equal(y, ry) and torch.equal(hl, rhl)


@pytest.mark.parametrize("disc", ("zoh", "euler"))
def test_graph_replay_fused_core(disc):
    import torch
    w = gen.SMALL.with_(name="graph_core", batch=2, seq_len=1300, d_inner=130, h0=True)
    inp = gen.generate(w)
    d = {k: dev(v) for k, v in inp.items()}
    y = torch.empty((w.M, w.d_inner), device="cuda")
    hl = torch.empty((w.batch, w.d_inner, w.d_state), device="cuda")
    _core(d, w, disc, y, hl)
    torch.cuda.synchronize()
    ey, ehl = y.clone(), hl.clone()
    oy, _, ohl = oracle.mamba1_core(inp["x"], inp["w_conv"], inp["b_conv"], inp["delta"],
                                    inp["A_log"], inp["B"], inp["C"], inp["D_vec"], inp["z"],
                                    inp["h0"], batch=w.batch, seq_len=w.seq_len, disc=disc,
                                    h_last=True)
    assert_close(host(ey), oy, "y (eager)")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _core(d, w, disc, y, hl)   # warm-up on the side stream, as capture requires
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _core(d, w, disc, y, hl)
    for r in range(REPLAYS):
        y.fill_(float("nan"))
        hl.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ey), f"replay {r}: y"
        assert torch.equal(hl, ehl), f"replay {r}: h_last"


@pytest.mark.parametrize("disc", ("zoh", "euler"))
def test_graph_replay_decode_steps(disc):
    """Eight decode steps captured as one graph: each replay, from the same
    carried state, equals the eager steps and the oracle."""
    import torch
    steps = 8
    w = gen.DECODE.with_(name="graph_decode", batch=16, d_inner=512, seq_len=steps)
    inp = gen.generate(w)
    d = {k: dev(v) for k, v in inp.items()}
    xs = [{k: d[k][s].clone() for k in ("x", "z", "delta", "B", "C")} for s in range(steps)]
    h0, cs0 = d["h"].clone(), d["conv_state"].clone()
    h, cs = h0.clone(), cs0.clone()
    ys = [torch.empty((w.batch, w.d_inner), device="cuda") for _ in range(steps)]

    def run():
        for s in range(steps):
            st = xs[s]
            mss.selective_step(st["x"], st["z"], st["delta"], d["A_log"], st["B"], st["C"],
                               d["D_vec"], d["w_conv"], d["b_conv"], cs, h, disc=disc,
                               out=ys[s])

    run()
    torch.cuda.synchronize()
    ey = [y.clone() for y in ys]
    eh, ecs = h.clone(), cs.clone()
    ocs, oh = inp["conv_state"].astype(np.float64), inp["h"].astype(np.float64)
    for s in range(steps):
        oy, ocs, oh = oracle.selective_step(inp["x"][s], inp["z"][s], inp["delta"][s],
                                            inp["A_log"], inp["B"][s], inp["C"][s],
                                            inp["D_vec"], inp["w_conv"], inp["b_conv"], ocs, oh,
                                            disc=disc)
        assert_close(host(ey[s]), oy, f"y step {s} (eager)")
    assert_close(host(eh), oh, "h (eager)")
    g = torch.cuda.CUDAGraph()
    h.copy_(h0)
    cs.copy_(cs0)
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        run()
    torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for r in range(REPLAYS):
        h.copy_(h0)
        cs.copy_(cs0)
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(ys[s], ey[s]), f"replay {r}: y step {s}"
        assert torch.equal(h, eh) and torch.equal(cs, ecs), f"replay {r}: state"


def test_graph_replay_scan_backward():
    """The scan backward (its workspace allocated before capture, its zeroing
    done by a fill kernel) replayed from a graph equals the eager call."""
    import torch
    w = gen.SMALL.with_(name="graph_bwd", batch=2, seq_len=700, d_inner=96, h0=True)
    inp = gen.generate(w)
    u = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=w.batch,
                           seq_len=w.seq_len).astype(np.float32)
    dout = gen.cotangent(w)
    d = {k: dev(v) for k, v in inp.items()}
    du_, dout_ = dev(u), dev(dout)
    nws = mss.workspace_bytes(mss.OP_SELECTIVE_SCAN_BACKWARD, batch=w.batch, seq_len=w.seq_len,
                              d_inner=w.d_inner, d_state=w.d_state)
    ws = torch.empty(nws + 256, dtype=torch.uint8, device="cuda")
    out = {}

    def run():
        out["g"] = mss.selective_scan_backward(du_, d["delta"], d["A_log"], d["B"], d["C"],
                                               d["D_vec"], d["z"], d["h0"], dout_,
                                               batch=w.batch, seq_len=w.seq_len, disc="zoh",
                                               need_dh0=True, workspace=ws)

    run()
    torch.cuda.synchronize()
    eg = {k: v.clone() for k, v in out["g"].items() if v is not None}
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        run()
    torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    graph_out = out["g"]
    for r in range(REPLAYS):
        for v in graph_out.values():
            if v is not None:
                v.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in eg.items():
            assert torch.equal(graph_out[k], v), f"replay {r}: {k}"
