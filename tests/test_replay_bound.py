"""What the scans' time split drops, on the CPU.

A segment that starts at t0 > 0 rebuilds its starting state by replaying the
recurrence from h = 0 at a step where every state has decayed by
2^-MSS_REPLAY_DECAY_BITS since (include/mss.h, "Time split").  These tests
take the fp64 oracle's states on the distribution of the 2.8B-class
workload (delta ~ N(-2, 0.5), A_log = log(n + 1)) and
  * check the closed form of the dropped part (replay_model.forward_dropped)
    against an explicit fp64 replay with the kernel's per-state start steps,
  * check the header's bound on it,
  * find how large an isolated input outlier just before a replay window
    must be before the dropped part reaches the 1e-4 tolerance.
The GPU side of the same question is tests/test_replay_outliers_gpu.py.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from mamba_selective_scan_causal_amd import inputs as gen
import replay_model as rm

CUT = rm.cut_bits_default()
W = gen.MAMBA_2P8B.with_(name="replay_tile", batch=1, seq_len=2048, d_inner=64, seed_index=41)
T0 = 1280          # a segment start (the 2.8B-class workload cuts 1280-step segments)
T_END = 1600


def _inputs():
    inp = gen.generate(W)
    u = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=1,
                           seq_len=W.seq_len).astype(np.float32)
    return inp, u


def _window(inp):
    A2 = rm.a2_of(inp["A_log"])
    dv32 = rm.softplus32(inp["delta"])
    return int(rm.forward_replay_starts(dv32, A2, T0, CUT).min())


def _run(inp, u, disc):
    y, hc, _ = oracle.selective_scan(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                     inp["D_vec"], inp["z"], None, batch=1, seq_len=W.seq_len,
                                     disc=disc, cols=np.arange(64), h_cache=True)
    E, dy, tw, join, hs = rm.forward_dropped(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                             inp["z"], L=W.seq_len, b=0, d0=0, t0=T0,
                                             t_end=T_END, h_true=hc, cut=CUT)
    return y, hc, E, dy, tw, join, hs


def _replay_fp64(inp, u, disc, join):
    """The kernel's algorithm in fp64: state n restarts from 0 at join[n] and
    runs the plain recurrence to T_END; returns y over [T0, T_END) (T, 64)."""
    A = -np.exp(np.clip(inp["A_log"].astype(np.float64), -10.0, 5.0))        # (64, N)
    dv = np.logaddexp(0.0, inp["delta"].astype(np.float64))                  # (L, 64)
    uu = u.astype(np.float64)
    Bm, Cm = inp["B"].astype(np.float64), inp["C"].astype(np.float64)
    N = A.shape[1]
    h = np.zeros((64, N))
    out = []
    for t in range(int(join.min()), T_END):
        x = dv[t][:, None] * A
        a = np.exp(x)
        bb = (np.expm1(x) / A) * Bm[t][None, :] if disc == "zoh" else dv[t][:, None] * Bm[t][None, :]
        live = (join <= t)[None, :]
        h = np.where(live, a * h + bb * uu[t][:, None], 0.0)
        if t >= T0:
            yv = inp["D_vec"].astype(np.float64) * uu[t] + (h * Cm[t][None, :]).sum(axis=1)
            zz = inp["z"][t].astype(np.float64)
            out.append(yv * zz / (1.0 + np.exp(-zz)))
    return np.array(out)


@pytest.mark.parametrize("disc", ("zoh", "euler"))
def test_dropped_part_closed_form(disc):
    """oracle y - modelled dropped part == an explicit replay with the
    kernel's start steps (fp64), to rounding."""
    inp, u = _inputs()
    y, _, _, dy, tw, join, _ = _run(inp, u, disc)
    assert 0 < tw < T0 - 64 and join.min() == tw and join.max() < T0
    emul = _replay_fp64(inp, u, disc, join)
    want = y[:, T0:T_END].T - dy
    assert np.max(np.abs(emul - want)) <= 1e-11 * np.max(np.abs(want))
    # and the dropped part is not zero: the closed form is what is compared
    assert np.max(np.abs(dy)) > 1e-12


@pytest.mark.parametrize("disc", ("zoh", "euler"))
@pytest.mark.parametrize("outlier", (1e3, 1e5))
def test_header_bound_holds(disc, outlier):
    """|dropped part of y_t| <= 2^-cut ||C_t||_1 |SiLU(z_t)| max_n |h_{tj_n - 1}[n]|,
    with an outlier row in u one step before the replay window."""
    inp, u = _inputs()
    tw = _window(inp)
    u[tw - 1] = outlier
    y, _, _, dy, tw2, _, hs = _run(inp, u, disc)
    assert tw2 == tw
    bound = rm.header_bound(hs, inp["C"][T0:T_END], inp["z"][T0:T_END], CUT)
    assert np.all(np.abs(dy) <= bound * (1 + 1e-9))
    # the outlier is what the replay start state carries
    assert np.abs(hs).max() > 0.1 * outlier * min(1.0, 1.0 / 16.0)


def _rel(dy, y):
    """The tests' metric on the segment's own outputs (steps >= t0): the
    outlier's own outputs, before the segment, are not in the rms."""
    yy = y[:, T0:T_END].T
    rms = np.sqrt(np.mean(yy * yy))
    return float(np.max(np.abs(dy) / np.maximum(np.abs(yy), rms)))


def _threshold(disc):
    inp, u0 = _inputs()
    tw = _window(inp)
    errs = {}
    for X in (1e2, 1e3, 1e4, 1e5, 1e6):
        u = u0.copy()
        u[tw - 1] = X
        y, _, _, dy, _, _, _ = _run(inp, u, disc)
        errs[X] = _rel(dy, y)
    return errs, 1e5 * 1e-4 / errs[1e5]


@pytest.mark.parametrize("disc", ("zoh", "euler"))
def test_outlier_size_that_reaches_the_tolerance(disc):
    """Relative error of the dropped part (the tests' metric, over the
    segment's outputs) against the size X of an outlier row in u one step
    before the earliest replay start: linear in X.  On these inputs 1e-4 is
    reached at X of a few 10^5 (typical |u| is ~0.5); where exactly depends
    on the data at the replay start (how much of the outlier the state
    there holds) -- the bound in terms of the state is the header's.
    MSS_FLAG_EXACT has no such limit.  A 2^-48 cut would stay below 1e-8
    at X = 1e6."""
    errs, threshold = _threshold(disc)
    for a, b in ((1e3, 1e4), (1e4, 1e5), (1e5, 1e6)):
        assert abs(errs[b] / errs[a] - 10.0) < 0.5, errs
    if CUT == 24:
        assert 1e4 < threshold < 1e7, (threshold, errs)
        assert errs[1e3] < 1e-5 and errs[1e6] > 1e-4, errs
    inp, u = _inputs()
    tw = _window(inp)
    u[tw - 1] = 1e6
    y, hc, _ = oracle.selective_scan(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                     inp["D_vec"], inp["z"], None, batch=1, seq_len=W.seq_len,
                                     disc=disc, cols=np.arange(64), h_cache=True)
    _, dy48, _, _, _ = rm.forward_dropped(u, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                          inp["z"], L=W.seq_len, b=0, d0=0, t0=T0, t_end=T_END,
                                          h_true=hc, cut=48)
    assert _rel(dy48, y) < 1e-8
