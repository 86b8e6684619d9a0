"""Large inputs just before a replay window, on the GPU.

The scans split time into segments; a segment rebuilds its starting state by
a replay whose start has decayed by 2^-MSS_REPLAY_DECAY_BITS (include/mss.h,
"Time split").  An outlier one step before that start is exactly what the
split drops (tests/replay_model.py, tests/test_replay_bound.py: at the
default 2^-24 an isolated outlier reaches 1e-4 at a few 10^5 on unit-scale
data).  Here, in the launch configuration of the benchmark-sized workloads:
  * outliers of 1e3 before a window: every entry point matches the oracle;
  * an outlier of 1e7: the forward scan's deviation from the oracle is the
    modelled dropped part, to rounding (and is above 1e-4: the bound bites);
  * MSS_FLAG_EXACT: outliers of 1e7 and 1e9 match the oracle.
Windows are located with the library's own split (mss_time_split) and the
replay rule restated in tests/replay_model.py."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
import mamba_selective_scan_causal_amd as mss
from mamba_selective_scan_causal_amd import inputs as gen
from gpu_util import announce, assert_close, dev, host, nan_like, rel_err
import replay_model as rm

pytestmark = pytest.mark.gpu

DISCS = ("zoh", "euler")
CUT = rm.cut_bits_default()


@pytest.fixture(autouse=True)
def _announce(request):
    announce(request.node.nodeid)
    yield


# ---- forward: the scan on a given u, one batch row of the 2.8B-class shape ----

WF = gen.MAMBA_2P8B.with_(name="outlier_fwd", batch=1, seed_index=51)
T0 = 1280


@functools.lru_cache(maxsize=1)
def _fwd_inputs():
    inp = gen.generate(WF)
    u = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=WF.batch,
                           seq_len=WF.seq_len).astype(np.float32)
    return inp, u


def _fwd_window(inp, t0):
    A2 = rm.a2_of(inp["A_log"][:64])
    dv32 = rm.softplus32(inp["delta"][:WF.seq_len, :64])
    return int(rm.forward_replay_starts(dv32, A2, t0, CUT).min())


def _scan(u, inp, disc, exact=False):
    import torch
    w = WF
    y = nan_like((w.M, w.d_inner))
    mss.selective_scan(dev(u), dev(inp["delta"]), dev(inp["A_log"]), dev(inp["B"]),
                       dev(inp["C"]), dev(inp["D_vec"]), dev(inp["z"]), None, batch=w.batch,
                       seq_len=w.seq_len, disc=disc, out=y, exact=exact)
    torch.cuda.synchronize()
    return host(y)


def _oracle_tile(u, inp, disc):
    y, hc, _ = oracle.selective_scan(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                     inp["D_vec"], inp["z"], None, batch=WF.batch,
                                     seq_len=WF.seq_len, disc=disc, cols=np.arange(64),
                                     h_cache=True)
    return y.T, hc          # y (L, 64)


def test_forward_segment_start_is_where_the_model_says():
    seg = mss.time_split(mss.OP_SELECTIVE_SCAN, batch=WF.batch, seq_len=WF.seq_len,
                         d_inner=WF.d_inner, d_state=WF.d_state, d_conv=WF.d_conv)
    assert T0 in rm.segment_starts(0, WF.seq_len, seg), seg
    inp, _ = _fwd_inputs()
    tw = _fwd_window(inp, T0)
    assert T0 - 400 < tw < T0 - 50


@pytest.mark.parametrize("disc", DISCS)
def test_scan_outlier_1e3_before_window(disc):
    inp, u0 = _fwd_inputs()
    tw = _fwd_window(inp, T0)
    u = u0.copy()
    u[tw - 1, :64] = 1e3
    y = _scan(u, inp, disc)
    oy, _ = _oracle_tile(u, inp, disc)
    assert_close(y[:, :64], oy, "y, tile 0")
    assert_close(y[T0:T0 + 400, :64], oy[T0:T0 + 400], "y, the segment's first 400 steps")


@pytest.mark.parametrize("disc", DISCS)
def test_scan_outlier_1e7_deviation_is_the_modelled_drop(disc):
    """Past the bound the default split deviates from the oracle, by exactly
    the part the model says it drops."""
    inp, u0 = _fwd_inputs()
    tw = _fwd_window(inp, T0)
    u = u0.copy()
    u[tw - 1, :64] = 1e7
    y = _scan(u, inp, disc)
    oy, hc = _oracle_tile(u, inp, disc)
    T1 = T0 + 400
    _, dy, tw2, _, _ = rm.forward_dropped(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                          inp["z"], L=WF.seq_len, b=0, d0=0, t0=T0, t_end=T1,
                                          h_true=hc, cut=CUT)
    assert tw2 == tw
    seg_y = oy[T0:T1]
    dev_ = y[T0:T1, :64] - seg_y
    if CUT == 24:
        assert rel_err(y[T0:T1, :64], seg_y) > 1e-4       # the bound bites
    # the GPU misses the modelled part, and nothing else (to fp32 rounding)
    rms = np.sqrt(np.mean(seg_y * seg_y))
    resid = np.abs(dev_ + dy) / np.maximum(np.abs(seg_y), rms)
    assert resid.max() <= 1e-5, resid.max()


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("X", (1e7, 1e9))
def test_scan_exact_flag_outlier(disc, X):
    inp, u0 = _fwd_inputs()
    tw = _fwd_window(inp, T0)
    u = u0.copy()
    u[tw - 1, :64] = X
    y = _scan(u, inp, disc, exact=True)
    oy, _ = _oracle_tile(u, inp, disc)
    assert_close(y[T0:T0 + 400, :64], oy[T0:T0 + 400], "y, the segment's first 400 steps")
    assert_close(y[:, :64], oy, "y, tile 0")


# ---- fused core at the benchmark's shape and launch configuration ----------

WC = gen.MAMBA_2P8B


@functools.lru_cache(maxsize=1)
def _core_inputs():
    return gen.generate(WC)


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("X,exact", ((1e3, False), (1e5, True)))
def test_core_x_outlier_before_window(disc, X, exact):
    import torch
    w = WC
    seg = mss.time_split(mss.OP_SELECTIVE_SCAN, batch=w.batch, seq_len=w.seq_len,
                         d_inner=w.d_inner, d_state=w.d_state, d_conv=w.d_conv)
    assert seg == 1280 and T0 in rm.segment_starts(0, w.seq_len, seg)
    inp = {k: v.copy() if k == "x" else v for k, v in _core_inputs().items()}
    A2 = rm.a2_of(inp["A_log"][:64])
    tw = int(rm.forward_replay_starts(rm.softplus32(inp["delta"][:w.seq_len, :64]), A2, T0,
                                      CUT).min())
    inp["x"][tw - 1, :64] = X
    y = nan_like((w.M, w.d_inner))
    d = {k: dev(v) for k, v in inp.items()}
    mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"], d["B"], d["C"],
                    d["D_vec"], d["z"], None, batch=w.batch, seq_len=w.seq_len, disc=disc, out=y,
                    exact=exact)
    torch.cuda.synchronize()
    g = host(y[:w.seq_len, :64]).T
    oy, _, _ = oracle.mamba1_core(inp["x"], inp["w_conv"], inp["b_conv"], inp["delta"],
                                  inp["A_log"], inp["B"], inp["C"], inp["D_vec"], inp["z"], None,
                                  batch=w.batch, seq_len=w.seq_len, disc=disc,
                                  cols=np.arange(64))
    assert_close(g[:, T0:T0 + 400], oy[:, T0:T0 + 400], "y, the segment's first 400 steps")
    assert_close(g, oy, "y, tile 0 of batch row 0")


# ---- scan backward: a u outlier before the forward replay window and a dout
# outlier just past the adjoint's replay window of the same segment --------

WB = gen.MAMBA_2P8B.with_(name="outlier_bwd", batch=1, seq_len=4096, d_inner=512,
                          seed_index=52)


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("X,exact", ((1e3, False), (1e5, True)))
def test_backward_outliers_around_a_segment(disc, X, exact):
    import torch
    w = WB
    seg = mss.time_split(mss.OP_SELECTIVE_SCAN_BACKWARD, batch=w.batch, seq_len=w.seq_len,
                         d_inner=w.d_inner, d_state=w.d_state)
    inp = gen.generate(w)
    u = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=1,
                           seq_len=w.seq_len).astype(np.float32)
    dout = gen.cotangent(w)
    A2 = rm.a2_of(inp["A_log"][:32])
    dv32 = rm.softplus32(inp["delta"][:, :32])
    mn = (-A2).min(axis=1)
    # the segment of tile 0 that starts at t0 and ends at t1
    t0 = 1280
    assert t0 in rm.segment_starts(0, w.seq_len, seg)
    t1 = min(t0 + seg, w.seq_len)
    tw, _ = rm.replay_start(dv32, mn, t0, CUT)
    te = rm.replay_end(dv32, mn, t1, CUT)
    assert 0 < tw < t0 and t1 < te < w.seq_len
    u[tw - 1, :32] = X
    dout[te, :32] = X
    d = {k: dev(v) for k, v in inp.items()}
    g = mss.selective_scan_backward(dev(u), d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"],
                                    d["z"], None, dev(dout), batch=1, seq_len=w.seq_len,
                                    disc=disc, exact=exact)
    torch.cuda.synchronize()
    og = oracle.selective_scan_backward(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                        inp["D_vec"], inp["z"], None, dout, batch=1,
                                        seq_len=w.seq_len, disc=disc)
    for k in ("du", "ddelta", "dz"):
        assert_close(host(g[k])[t0:t1, :32], og[k][t0:t1, :32], f"{k}, the segment")
    for k in ("du", "ddelta", "dA_log", "dB", "dC", "dD", "dz"):
        assert_close(host(g[k]), og[k], k)


# ---- Mamba-2 SSD scan: an x outlier before a segment's replay chunk --------

WS = gen.SSD_2P7B


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("X,exact", ((1e3, False), (1e5, True)))
def test_ssd_x_outlier_before_window(disc, X, exact):
    import torch
    w = WS
    seg = mss.ssd_time_split(batch=w.batch, seq_len=w.seq_len, n_heads=w.n_heads,
                             head_dim=w.head_dim, d_state=w.d_state, n_groups=w.n_groups)
    assert seg == 2048
    inp = gen.generate_ssd(w)
    h, P, Q = 0, w.head_dim, 32
    t0 = seg
    A = -np.exp(np.clip(float(inp["A_log"][h]), -10.0, 5.0))
    dv = np.logaddexp(0.0, inp["dt"][:w.seq_len, h].astype(np.float64) + inp["dt_bias"][h])
    s, tw = 0.0, 0
    for tt in range(t0 - 1, -1, -1):
        s += dv[tt] * -A * 1.4426950408889634
        if s >= CUT:
            tw = tt
            break
    cw = tw // Q * Q
    assert 0 < cw < t0
    inp["x"][cw - 1, h * P:(h + 1) * P] = X
    d = {k: dev(v) for k, v in inp.items()}
    y = nan_like((w.M, w.n_heads * P))
    mss.ssd_scan(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D_vec"], d["dt_bias"], None,
                 batch=w.batch, seq_len=w.seq_len, head_dim=P, d_state=w.d_state,
                 n_groups=w.n_groups, disc=disc, out=y, exact=exact)
    torch.cuda.synchronize()
    hs = [h, 1]
    cols = np.concatenate([np.arange(k * P, (k + 1) * P) for k in hs])
    oy, _ = oracle.ssd_scan(np.ascontiguousarray(inp["x"][:, cols]),
                            np.ascontiguousarray(inp["dt"][:, hs]), inp["A_log"][hs], inp["B"],
                            inp["C"], inp["D_vec"][hs], inp["dt_bias"][hs], None, batch=w.batch,
                            seq_len=w.seq_len, n_heads=len(hs), head_dim=P, d_state=w.d_state,
                            n_groups=w.n_groups, disc=disc)
    g = host(y[:, cols])
    assert_close(g[t0:t0 + 256, :P], oy[t0:t0 + 256, :P], "y, head 0, the segment's start")
    assert_close(g, oy, "y, heads 0-1")
