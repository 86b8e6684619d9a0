"""CPU model of what the time split of the scans leaves out, for tests.

The HIP scans process time in segments; a segment that starts at t0 > 0
rebuilds its starting state from the steps before it, going back only until
their weight has decayed below 2^-cut.  Where each state's replay starts is
a rule on fp32 decay products or sums of softplus(delta) (the kernels' own
rules, restated here in numpy), and what it drops is a closed form of the
fp64 oracle's states:

    state n of column d at t >= t0 lacks  E_n(t) = prod_{s=tj_n..t} aBar_s[n] * h_{tj_n - 1}[n]

where tj_n is the step the replay of state n started from, and y_t lacks
SiLU(z_t) * sum_n C_t[n] E_n(t).  (A state that never had a replay start,
tj_n = 0, is exact.)  The backward's adjoint replay is the mirror image: the
adjoint entering a segment's last step t1 - 1 is rebuilt from g = 0 at a step
te found by walking delta forward from t1.

The fp32 decisions of this model may differ from the kernel's by a step where
a sum sits within rounding of the bound; the dropped magnitudes do not depend
on that.  Only tests import this module.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = np.float32(1.4426950408889634)
SMALL_X2 = np.float32(0.015625) * LOG2E      # |dv A| = 2^-6 in log2 units
BLOCK = 8                                      # the forward kernel's straight-line block
TILE_FWD = 64
TILE_BWD = 32


def softplus32(x) -> np.ndarray:
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64)).astype(np.float32)


def a2_of(A_log) -> np.ndarray:
    """A * log2(e) in fp32, as the kernels hold it: (D, N)."""
    A = -np.exp(np.clip(np.asarray(A_log, dtype=np.float32), -10.0, 5.0)).astype(np.float32)
    return (A * LOG2E).astype(np.float32)


def segment_starts(tile: int, L: int, seg: int):
    """Steps t0 in (0, L) of `tile` at which a segment of the flattened
    (tile, t) space starts (the split that mss_time_split reports: tiles
    padded to a multiple of 8 steps)."""
    Lp = (L + 7) // 8 * 8
    first = (-tile * Lp) % seg
    return [t for t in range(first, L, seg) if t > 0]


def replay_start(dv32: np.ndarray, min_a2: np.ndarray, t0: int, cut: float):
    """The scan backward's forward-state replay (and the SSD scan's, per
    head): backward walk from t0 - 1 to the first step tt at which
    S = sum_{s=tt}^{t0-1} dv_s satisfies S * min_a2 >= cut in every lane,
    or 0.  dv32: (L, lanes) fp32; min_a2: (lanes,) fp32.  Returns (tt, S)."""
    S = np.zeros(dv32.shape[1], dtype=np.float32)
    for tt in range(t0 - 1, -1, -1):
        S = (S + dv32[tt]).astype(np.float32)
        if np.all(S * min_a2 >= np.float32(cut)):
            return tt, S
    return 0, S


def replay_end(dv32: np.ndarray, min_a2: np.ndarray, t1: int, cut: float) -> int:
    """Forward walk from t1 (the backward's adjoint replay): one past the
    first step tt at which sum_{s=t1}^{tt} dv_s * min_a2 >= cut in every
    lane, or L."""
    L = dv32.shape[0]
    S = np.zeros(dv32.shape[1], dtype=np.float32)
    for tt in range(t1, L):
        S = (S + dv32[tt]).astype(np.float32)
        if np.all(S * min_a2 >= np.float32(cut)):
            return tt + 1
    return L


def forward_replay_starts(dv32: np.ndarray, A2: np.ndarray, t0: int, cut: float) -> np.ndarray:
    """First step of every state's replay (N,) in the forward kernel: the
    kernel accumulates the state entering t0 newest step first, in blocks of
    8 counted back from t0, keeping the decay to t0 as a running fp32
    product q; state n stops after the first block (short of t = 0) at whose
    start q_n < 2^-cut in every lane.  States that never stop start at 0."""
    lanes, N = A2.shape
    q = np.ones((lanes, N), dtype=np.float32)
    thr = np.float32(2.0 ** -cut)
    start = np.zeros(N, dtype=np.int64)
    active = np.ones(N, dtype=bool)
    tb = t0 - BLOCK
    while True:
        for i in range(BLOCK - 1, -1, -1):
            t = tb + i
            if t < 0:
                continue
            a = np.exp2((dv32[t][:, None] * A2).astype(np.float32)).astype(np.float32)
            q[:, active] = (q[:, active] * a[:, active]).astype(np.float32)
        if tb <= 0:
            break
        for n in range(N):
            if active[n] and np.all(q[:, n] < thr):
                active[n] = False
                start[n] = tb
        if not active.any():
            break
        tb -= BLOCK
    start[active] = 0
    return start


def forward_dropped(u, delta, A_log, B, C, z, *, L: int, b: int, d0: int, t0: int,
                    t_end: int, h_true: np.ndarray, cut: float):
    """The forward kernel's dropped part for the segment of the 64-channel
    tile starting at channel d0 of batch row b that begins at t0, over steps
    [t0, t_end).  h_true: fp64 oracle states (64, L, N) of those channels
    (h after the update of each step).  Returns (E, dy, tw, join, hstart):
    E (64, t_end - t0, N) what the kernel's states lack, dy (t_end - t0, 64)
    what its y lacks, tw the replay start, join (N,) the replay start of each
    state and hstart (64, N) the oracle state each replay starts from (0 for
    a replay from t = 0).
    """
    rows = slice(b * L, (b + 1) * L)
    cols = slice(d0, d0 + TILE_FWD)
    A2 = a2_of(A_log[cols])                        # (64, N)
    dv32 = softplus32(delta[rows, cols])          # (L, 64)
    dv64 = np.logaddexp(0.0, delta[rows, cols].astype(np.float64))
    join = forward_replay_starts(dv32, A2, t0, cut)
    tw = int(join.min())
    A = -np.exp(np.clip(A_log[cols].astype(np.float64), -10.0, 5.0))   # (64, N)
    T = t_end - t0
    E = np.zeros((TILE_FWD, T, A.shape[1]))
    hs = np.zeros((TILE_FWD, A.shape[1]))
    csum = np.concatenate([np.zeros((1, TILE_FWD)), np.cumsum(dv64, axis=0)])   # (L+1, 64)
    for n in range(A.shape[1]):
        tj = int(join[n])
        if tj == 0:
            continue
        hstart = h_true[:, tj - 1, n]                                   # (64,)
        hs[:, n] = hstart
        span = csum[t0 + 1:t_end + 1] - csum[tj]                        # (T, 64): sum dv over [tj, t]
        E[:, :, n] = (np.exp(A[:, n][None, :] * span) * hstart[None, :]).T
    Cr = C[rows][t0:t_end].astype(np.float64)                            # (T, N)
    dy = np.einsum("dtn,tn->td", E, Cr)
    if z is not None:
        zz = z[rows, cols][t0:t_end].astype(np.float64)
        dy = dy * (zz / (1.0 + np.exp(-zz)))
    return E, dy, tw, join, hs


def header_bound(hstart: np.ndarray, C_rows, z_rows, cut: float) -> np.ndarray:
    """The bound the header states for y_t: 2^-cut * ||C_t||_1 * |SiLU(z_t)|
    * max_n |h_{tj_n - 1}[n]|, per (t, channel); hstart (64, N)."""
    hmax = np.abs(hstart).max(axis=1)                                  # (64,)
    c1 = np.abs(np.asarray(C_rows, dtype=np.float64)).sum(axis=1)     # (T,)
    g = np.ones_like(c1)[:, None]
    if z_rows is not None:
        zz = np.asarray(z_rows, dtype=np.float64)
        g = np.abs(zz / (1.0 + np.exp(-zz)))
    return (2.0 ** -cut) * c1[:, None] * g * hmax[None, :]


def cut_bits_default() -> int:
    """MSS_REPLAY_DECAY_BITS as include/mss.h defines it."""
    import os
    import re
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                       "mss.h")
    m = re.search(r"#define MSS_REPLAY_DECAY_BITS (\d+)", open(hdr).read())
    return int(m.group(1))


def ln2_window(cut: float, A_min: float, dv_mean: float) -> float:
    """Expected replay window in steps for a slowest |A| and mean dv."""
    return cut * math.log(2.0) / (A_min * dv_mean)
