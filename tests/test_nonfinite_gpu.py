"""Non-finite inputs on the GPU.  NaN and Inf inputs are outside the contract
(their outputs are unspecified), but a call that receives them must return
and must not spread them: every output the fp64 oracle computes as finite
from the same inputs must be finite and within the usual 1e-4 of it
(gpu_util.rel_err compares only where the oracle is finite and counts a
non-finite GPU value there as an infinite error).

Every data-dependent loop in the kernels (the decay-bounded replay walks)
is bounded by the sequence ends, so a NaN that stops a walk from ever
reaching its decay bound only lengthens it."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import mamba_selective_scan_causal_amd as mss
from mamba_selective_scan_causal_amd import inputs as gen
from gpu_util import announce, assert_close, dev, host, nan_like

pytestmark = pytest.mark.gpu

DISCS = ("zoh", "euler")


@pytest.fixture(autouse=True)
def _announce(request):
    announce(request.node.nodeid)
    yield


W = gen.SMALL.with_(name="nonfinite", batch=2, seq_len=1500, d_inner=100, h0=True)


def _poison(inp, w):
    """A NaN in delta (row 0, t = 700, channel 37), +Inf in x (row 1, t = 40,
    channel 5), -Inf in z (row 0, t = 1200, channel 60)."""
    L = w.seq_len
    inp["delta"][0 * L + 700, 37] = np.nan
    inp["x"][1 * L + 40, 5] = np.inf
    inp["z"][0 * L + 1200, 60] = -np.inf
    return inp


@pytest.mark.parametrize("disc", DISCS)
def test_core_contains_nonfinite_inputs(disc):
    import torch
    w = W
    inp = _poison(gen.generate(w), w)
    d = {k: dev(v) for k, v in inp.items()}
    B, L, D, N = w.batch, w.seq_len, w.d_inner, w.d_state
    y, hl = nan_like((B * L, D)), nan_like((B, D, N))
    mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"], d["B"], d["C"],
                    d["D_vec"], d["z"], d["h0"], batch=B, seq_len=L, disc=disc, h_last=hl, out=y)
    torch.cuda.synchronize()
    oy, _, ohl = oracle.mamba1_core(inp["x"], inp["w_conv"], inp["b_conv"], inp["delta"],
                                    inp["A_log"], inp["B"], inp["C"], inp["D_vec"], inp["z"],
                                    inp["h0"], batch=B, seq_len=L, disc=disc, h_last=True)
    # the poisoned channels are non-finite in the oracle from the poisoned
    # step on; everything else is finite and must match
    assert not np.isfinite(oy[700:L, 37]).any() and np.isfinite(oy[:700, 37]).all()
    assert np.isfinite(oy).sum() > 0.99 * oy.size
    assert_close(host(y), oy, "y")
    assert_close(host(hl), ohl, "h_last")


@pytest.mark.parametrize("disc", DISCS)
def test_core_infinite_delta_inside_a_replay_window(disc):
    """+Inf in delta a few steps before a segment start, so dv = +Inf lies
    inside the window the segment replays; aBar = 0 there ends the replay's
    decay product, and every state must still be rebuilt correctly.  The
    segment starts of batch row 1's two channel tiles come from the
    library's own split (mss_time_split).  ZOH: aBar = 0 resets the column
    there and every output stays finite; EULER: dv B u is infinite, the
    column is non-finite from there on.  Outputs are compared wherever the
    oracle is finite."""
    import torch
    import replay_model as rm
    w = W
    inp = gen.generate(w)
    L = w.seq_len
    seg = mss.time_split(mss.OP_SELECTIVE_SCAN, batch=w.batch, seq_len=L, d_inner=w.d_inner,
                         d_state=w.d_state, d_conv=w.d_conv)
    tiles = (w.d_inner + 63) // 64
    s_lo = [t for t in rm.segment_starts(1 * tiles + 0, L, seg) if t > 200]
    s_hi = [t for t in rm.segment_starts(1 * tiles + 1, L, seg) if t > 200]
    marks = ((s_hi[6] - 4, 70), (s_hi[14] - 7, 99), (s_lo[5] - 4, 5))
    for t, ch in marks:
        inp["delta"][1 * L + t, ch] = np.inf
    d = {k: dev(v) for k, v in inp.items()}
    B, D, N = w.batch, w.d_inner, w.d_state
    y, hl = nan_like((B * L, D)), nan_like((B, D, N))
    mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"], d["B"], d["C"],
                    d["D_vec"], d["z"], d["h0"], batch=B, seq_len=L, disc=disc, h_last=hl, out=y)
    torch.cuda.synchronize()
    oy, _, ohl = oracle.mamba1_core(inp["x"], inp["w_conv"], inp["b_conv"], inp["delta"],
                                    inp["A_log"], inp["B"], inp["C"], inp["D_vec"], inp["z"],
                                    inp["h0"], batch=B, seq_len=L, disc=disc, h_last=True)
    if disc == "zoh":
        assert np.isfinite(oy).all()
    assert_close(host(y), oy, "y")
    assert_close(host(hl), ohl, "h_last")


@pytest.mark.parametrize("disc", DISCS)
def test_decode_step_contains_nonfinite_inputs(disc):
    import torch
    w = gen.DECODE.with_(name="nonfinite_decode", batch=8, d_inner=256, seq_len=3)
    inp = gen.generate(w)
    inp["x"][1, 3, 17] = np.nan       # step 1, sequence 3, channel 17
    inp["delta"][0, 6, 200] = np.inf
    d = {k: dev(v) for k, v in inp.items()}
    cs, h = d["conv_state"].clone(), d["h"].clone()
    ocs, oh = inp["conv_state"].astype(np.float64), inp["h"].astype(np.float64)
    for s in range(w.seq_len):
        st = {k: d[k][s].clone() for k in ("x", "z", "delta", "B", "C")}
        y = mss.selective_step(st["x"], st["z"], st["delta"], d["A_log"], st["B"], st["C"],
                               d["D_vec"], d["w_conv"], d["b_conv"], cs, h, disc=disc)
        torch.cuda.synchronize()
        oy, ocs, oh = oracle.selective_step(inp["x"][s], inp["z"][s], inp["delta"][s],
                                            inp["A_log"], inp["B"][s], inp["C"][s],
                                            inp["D_vec"], inp["w_conv"], inp["b_conv"], ocs, oh,
                                            disc=disc)
        assert_close(host(y), oy, f"y step {s}")
    assert not np.isfinite(oh[3, 17]).all()
    assert_close(host(h), oh, "h")
    assert_close(host(cs), ocs, "conv_state")


def test_scan_backward_contains_nonfinite_inputs():
    """A NaN in dout: gradients the oracle finds finite (all but the poisoned
    channel's steps up to the NaN, the dB / dC rows there and that channel's
    parameter sums) match."""
    import torch
    w = W.with_(seq_len=900)
    inp = gen.generate(w)
    u = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=w.batch,
                           seq_len=w.seq_len).astype(np.float32)
    dout = gen.cotangent(w)
    dout[1 * w.seq_len + 500, 11] = np.nan
    d = {k: dev(v) for k, v in inp.items()}
    g = mss.selective_scan_backward(dev(u), d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"],
                                    d["z"], d["h0"], dev(dout), batch=w.batch, seq_len=w.seq_len,
                                    disc="zoh", need_dh0=True)
    torch.cuda.synchronize()
    og = oracle.selective_scan_backward(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                        inp["D_vec"], inp["z"], inp["h0"], dout, batch=w.batch,
                                        seq_len=w.seq_len, disc="zoh")
    assert not np.isfinite(og["du"][w.seq_len + 500, 11])
    for k in ("du", "ddelta", "dA_log", "dB", "dC", "dD", "dz", "dh0"):
        assert_close(host(g[k]), og[k], k)


def test_ssd_contains_nonfinite_inputs():
    """NaN in dt and in B.  (A non-finite x is not covered: in the chunked
    form the masked-out entries of L o C B^T are exact zeros that still
    multiply every x of the chunk, so 0 * Inf can reach the chunk's earlier
    outputs of that column.)"""
    import torch
    w = gen.SSD_SMALL.with_(name="nonfinite_ssd", seq_len=700, n_heads=4, h0=True)
    inp = gen.generate_ssd(w)
    H, P = w.n_heads, w.head_dim
    inp["dt"][0 * w.seq_len + 300, 2] = np.nan                # row 0, head 2
    inp["B"][1 * w.seq_len + 650, 5] = np.nan                  # row 1, all heads
    d = {k: dev(v) for k, v in inp.items()}
    y, hl = nan_like((w.M, H * P)), nan_like((w.batch, H, P, w.d_state))
    mss.ssd_scan(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D_vec"], d["dt_bias"], d["h0"],
                 batch=w.batch, seq_len=w.seq_len, head_dim=P, d_state=w.d_state,
                 n_groups=w.n_groups, disc="zoh", h_last=hl, out=y)
    torch.cuda.synchronize()
    oy, ohl = oracle.ssd_scan(inp["x"], inp["dt"], inp["A_log"], inp["B"], inp["C"],
                              inp["D_vec"], inp["dt_bias"], inp["h0"], batch=w.batch,
                              seq_len=w.seq_len, n_heads=H, head_dim=P, d_state=w.d_state,
                              n_groups=w.n_groups, disc="zoh", h_last=True)
    assert not np.isfinite(oy[300:w.seq_len, 2 * P:3 * P]).all()
    assert np.isfinite(oy[:w.seq_len, 3 * P:]).all()
    assert not np.isfinite(oy[w.seq_len + 650:, :]).all()
    assert_close(host(y), oy, "y")
    assert_close(host(hl), ohl, "h_last")


@pytest.mark.parametrize("K", (3, 8))
def test_conv_contains_nonfinite_inputs(K):
    """+Inf and NaN in x with d_conv = 3 and 8, forward and backward of the
    conv1d + SiLU on their own: only the K taps of the method may meet a
    poisoned input, so outputs K or more steps after it (forward) or before
    it (dx) stay finite and match the oracle.  +Inf also sits at the last
    step of row 1, where a window running past the sequence end would meet
    it again."""
    import torch
    w = gen.SMALL.with_(name=f"nonfinite_conv_k{K}", batch=2, seq_len=300, d_inner=100,
                        d_conv=K, b_conv="normal")
    inp = gen.generate(w)
    L = w.seq_len
    inp["x"][0 * L + 100, 7] = np.inf
    inp["x"][0 * L + 200, 70] = np.nan
    inp["x"][1 * L + L - 1, 30] = np.inf
    d = {k: dev(v) for k, v in inp.items()}
    u = mss.conv1d_silu(d["x"], d["w_conv"], d["b_conv"], batch=w.batch, seq_len=L)
    torch.cuda.synchronize()
    ou = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=w.batch, seq_len=L)
    assert np.isfinite(ou[100 + K:L, 7]).all() and np.isfinite(ou[200 + K:L, 70]).all()
    assert_close(host(u), ou, "u")
    du = gen.cotangent(w)
    gx, gw, gb = mss.conv1d_silu_backward(d["x"], d["w_conv"], d["b_conv"], dev(du),
                                          batch=w.batch, seq_len=L)
    torch.cuda.synchronize()
    ox, ow, ob = oracle.conv1d_silu_backward(inp["x"], inp["w_conv"], inp["b_conv"], du,
                                             batch=w.batch, seq_len=L)
    assert np.isfinite(ox[:100 - K, 7]).all() and np.isfinite(ox[L:2 * L - K, 30]).all()
    assert np.isfinite(ox).sum() > 0.99 * ox.size
    for name, got, want in (("dx", gx, ox), ("dw", gw, ow), ("db", gb, ob)):
        assert_close(host(got), want, name)
