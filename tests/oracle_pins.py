"""Pins for the CPU oracle: checks against facts that do not come from it.

Each ``pin_*`` takes an object with the oracle's API (``oracle.Bound``) and
raises AssertionError when the oracle disagrees with:
  * a library routine (numpy.convolve, numpy.logaddexp, scipy expit, scipy expm),
  * an exact solution (the zero-order-hold step is the exact flow of
    dh/dt = A h + B u over a time dv with u held constant, computed here from
    the augmented matrix exponential; constant input gives a closed form),
  * brute force (the unrolled O(L^2) sum of decayed inputs),
  * or an invariant stated by the pages or fixed by the maths (causality,
    A_log clamp invariance, linearity, batch independence, determinism).

The same pins run against deliberately broken builds of the oracle to show
that each plausible mistake fails at least one of them.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import expm
from scipy.special import expit

ZOH, EULER = "zoh", "euler"


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _silu(v):
    return v * expit(v)


def _softplus(v):
    return np.logaddexp(0.0, v)


def _close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} off; worst abs err "
                           f"{err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")


def _zoh_flow(A, dv, h, w):
    """Exact state after time dv of dh/dt = A h + w from h (scalar A, w)."""
    M = np.array([[A * dv, w * dv], [0.0, 0.0]])
    E = expm(M)
    return E[0, 0] * h + E[0, 1]


def _scan_inputs(seed, B, L, D, N, *, alog_lo=-4.0, alog_hi=3.0, delta_mu=-1.0):
    g = _rng(seed)
    return dict(
        u=_f32(g.standard_normal((B * L, D))),
        delta=_f32(g.standard_normal((B * L, D)) + delta_mu),
        A_log=_f32(g.uniform(alog_lo, alog_hi, (D, N))),
        B=_f32(g.standard_normal((B * L, N))),
        C=_f32(g.standard_normal((B * L, N))),
        D_vec=_f32(g.uniform(0.5, 1.5, D)),
        z=_f32(g.standard_normal((B * L, D))),
        h0=_f32(0.3 * g.standard_normal((B, D, N))),
    )


# --------------------------------------------------------------------------
# conv1d + SiLU


def pin_conv_matches_numpy_convolve(orc):
    g = _rng(1)
    B, L, D = 3, 37, 5
    for K in (1, 2, 3, 4, 7):
        x = _f32(g.standard_normal((B * L, D)))
        w = _f32(0.5 * g.standard_normal((D, K)))
        bias = _f32(0.5 * g.standard_normal(D))
        u = orc.conv1d_silu(x, w, bias, batch=B, seq_len=L)
        xs = x.astype(np.float64).reshape(B, L, D)
        want = np.empty((B, L, D))
        for b in range(B):
            for d in range(D):
                # full-mode convolution sum_k x[t-k] w[k]; first L outputs are causal
                want[b, :, d] = np.convolve(xs[b, :, d], w[d].astype(np.float64))[:L] + bias[d]
        _close(u, _silu(want).reshape(B * L, D), 1e-12, 1e-300, f"conv K={K}")


def pin_conv_impulse_and_batch_edge(orc):
    g = _rng(2)
    B, L, D, K = 2, 10, 3, 4
    w = _f32(g.standard_normal((D, K)))
    bias = _f32(g.standard_normal(D))
    x = np.zeros((B * L, D), dtype=np.float32)
    x[L - 2, :] = 1.0  # impulse at t = L-2 of batch 0
    u = orc.conv1d_silu(x, w, bias, batch=B, seq_len=L).reshape(B, L, D)
    base = _silu(bias.astype(np.float64))
    want = np.broadcast_to(base, (B, L, D)).copy()
    want[0, L - 2] = _silu(bias.astype(np.float64) + w[:, 0])
    want[0, L - 1] = _silu(bias.astype(np.float64) + w[:, 1])
    _close(u, want, 1e-14, 0.0, "impulse")


def pin_short_sequence_shorter_than_kernel(orc):
    g = _rng(3)
    B, L, D, K = 2, 2, 4, 4
    x = _f32(g.standard_normal((B * L, D)))
    w = _f32(g.standard_normal((D, K)))
    u = orc.conv1d_silu(x, w, None, batch=B, seq_len=L).reshape(B, L, D)
    xs = x.astype(np.float64).reshape(B, L, D)
    want = np.stack([w[:, 0] * xs[:, 0], w[:, 0] * xs[:, 1] + w[:, 1] * xs[:, 0]], axis=1)
    _close(u, _silu(want), 1e-14, 0.0, "L<K")


# --------------------------------------------------------------------------
# softplus, gate, L = 1 closed forms


def pin_softplus_matches_logaddexp(orc):
    D = 401
    delta = _f32(np.linspace(-40.0, 40.0, D)).reshape(1, D)
    one = np.ones((1, D), dtype=np.float32)
    y, _, _ = orc.selective_scan(one, delta, np.zeros((D, 1), np.float32), np.ones((1, 1), np.float32),
                                 np.ones((1, 1), np.float32), None, None, None,
                                 batch=1, seq_len=1, disc=EULER)
    # L = 1 from h = 0 under EULER: h = dv * B * u = dv, y = C * h = dv
    _close(y, _softplus(delta.astype(np.float64)), 1e-14, 0.0, "softplus")


def pin_gate_and_skip(orc):
    D = 301
    z = _f32(np.linspace(-30.0, 30.0, D)).reshape(1, D)
    u = _f32(np.linspace(-2.0, 2.0, D)).reshape(1, D)
    dvec = _f32(np.linspace(0.5, 1.5, D))
    zeros_row = np.zeros((1, 2), np.float32)
    y, _, _ = orc.selective_scan(u, np.zeros((1, D), np.float32), np.zeros((D, 2), np.float32),
                                 zeros_row, zeros_row, dvec, z, None, batch=1, seq_len=1, disc=ZOH)
    want = dvec.astype(np.float64) * u.astype(np.float64) * _silu(z.astype(np.float64))
    _close(y, want, 1e-14, 0.0, "gate")


def pin_zoh_is_exact_flow(orc):
    """ZOH one step == exact ODE flow, for many (A, dv) incl. tiny dv*A."""
    g = _rng(4)
    D, N = 48, 4
    inp = _scan_inputs(4, 1, 1, D, N, alog_lo=-9.5, alog_hi=4.5, delta_mu=0.0)
    inp["delta"] = _f32(np.concatenate([g.normal(0, 3, D - 8), [-20, -15, -10, 0, 5, 10, 20, 30]])
                        ).reshape(1, D)
    _, _, hl = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], None,
                                  None, inp["h0"], batch=1, seq_len=1, disc=ZOH, h_last=True)
    A = -np.exp(inp["A_log"].astype(np.float64))
    dv = _softplus(inp["delta"][0].astype(np.float64))
    want = np.empty((D, N))
    for d in range(D):
        for n in range(N):
            w = float(inp["B"][0, n]) * float(inp["u"][0, d])
            want[d, n] = _zoh_flow(A[d, n], dv[d], float(inp["h0"][0, d, n]), w)
    _close(hl[0], want, 1e-11, 1e-300, "zoh flow")


def pin_euler_relation_to_zoh(orc):
    """From h = 0 after one step: h_zoh = h_euler * expm1(x)/x with x = dv*A, and
    h_euler = softplus(delta) * B * u."""
    D, N = 64, 4
    inp = _scan_inputs(5, 1, 1, D, N, alog_lo=-9.5, alog_hi=4.5, delta_mu=-2.0)
    kw = dict(batch=1, seq_len=1, h_last=True)
    _, _, hz = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], **kw,
                                  disc=ZOH)
    _, _, he = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], **kw,
                                  disc=EULER)
    dv = _softplus(inp["delta"][0].astype(np.float64))
    want_e = dv[:, None] * inp["B"][0].astype(np.float64)[None, :] * \
        inp["u"][0].astype(np.float64)[:, None]
    _close(he[0], want_e, 1e-14, 1e-300, "euler")
    x = dv[:, None] * -np.exp(inp["A_log"].astype(np.float64))
    _close(hz[0], he[0] * (np.expm1(x) / x), 1e-13, 1e-300, "zoh/euler ratio")


def pin_modes_agree_for_tiny_step(orc):
    inp = _scan_inputs(6, 2, 16, 8, 4)
    inp["delta"] = np.full_like(inp["delta"], -20.0)
    kw = dict(batch=2, seq_len=16, h_cache=True)
    yz, hz, _ = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                   inp["D_vec"], inp["z"], **kw, disc=ZOH)
    ye, he, _ = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                   inp["D_vec"], inp["z"], **kw, disc=EULER)
    # bBar_zoh / bBar_euler = expm1(x)/x = 1 + x/2 + ..., |x| = dv|A| <= 2e-9 * e^3
    _close(hz, he, 1e-7, 1e-7 * np.abs(he).max(), "modes at dv~2e-9")
    _close(yz, ye, 1e-7, 1e-7 * np.abs(ye).max(), "modes at dv~2e-9 (y)")


# --------------------------------------------------------------------------
# the recurrence


def pin_constant_input_closed_form(orc):
    """Constant dv, u, B, C: ZOH h_t = -(B u / A)(1 - exp(A dv (t+1))) (exact flow
    over time (t+1) dv); EULER h_t = dv B u (1 - a^(t+1)) / (1 - a)."""
    L, D, N = 50, 6, 3
    g = _rng(7)
    alog = _f32(g.uniform(-3.0, 2.0, (D, N)))
    dl = _f32(g.normal(-1.0, 1.0, D))
    uval = _f32(g.normal(0, 1, D))
    bval = _f32(g.normal(0, 1, N))
    cval = _f32(g.normal(0, 1, N))
    u = np.broadcast_to(uval, (L, D)).copy()
    delta = np.broadcast_to(dl, (L, D)).copy()
    Bm = np.broadcast_to(bval, (L, N)).copy()
    Cm = np.broadcast_to(cval, (L, N)).copy()
    dvec = _f32(g.uniform(0.5, 1.5, D))
    A = -np.exp(alog.astype(np.float64))
    dv = _softplus(dl.astype(np.float64))
    t1 = np.arange(1, L + 1, dtype=np.float64)[:, None, None]
    Bu = uval.astype(np.float64)[:, None] * bval.astype(np.float64)[None, :]
    for disc in (ZOH, EULER):
        y, hc, _ = orc.selective_scan(u, delta, alog, Bm, Cm, dvec, None, None, batch=1, seq_len=L,
                                      disc=disc, h_cache=True)
        if disc == ZOH:
            want = -(Bu / A)[None] * (-np.expm1(A[None] * dv[None, :, None] * t1))
        else:
            a = np.exp(A * dv[:, None])
            want = (dv[:, None] * Bu)[None] * (1 - a[None] ** t1) / (1 - a[None])
        _close(hc[0], want, 1e-11, 1e-300, f"geometric {disc}")
        wy = dvec.astype(np.float64) * uval.astype(np.float64) + want @ cval.astype(np.float64)
        _close(y, wy, 1e-11, 1e-12, f"geometric y {disc}")


def _bruteforce(u, delta, A_log, Bm, Cm, dvec, z, h0, B, L, disc):
    """Unrolled h_t = (prod_{r<=t} a_r) h0 + sum_{s<=t} (prod_{r=s+1..t} a_r) b_s u_s."""
    D, N = A_log.shape
    A = -np.exp(A_log.astype(np.float64))
    u = u.astype(np.float64).reshape(B, L, D)
    dv = _softplus(delta.astype(np.float64)).reshape(B, L, D)
    Bm = Bm.astype(np.float64).reshape(B, L, N)
    Cm = Cm.astype(np.float64).reshape(B, L, N)
    H = np.zeros((B, L, D, N))
    for b in range(B):
        a = np.exp(dv[b][:, :, None] * A[None])                        # (L, D, N)
        if disc == ZOH:
            # input part of the exact flow over each step (h = 0 start)
            inc = np.empty((L, D, N))
            for t in range(L):
                for d in range(D):
                    for n in range(N):
                        inc[t, d, n] = _zoh_flow(A[d, n], dv[b, t, d], 0.0,
                                                 Bm[b, t, n] * u[b, t, d])
        else:
            inc = dv[b][:, :, None] * Bm[b][:, None, :] * u[b][:, :, None]
        for t in range(L):
            acc = np.prod(a[: t + 1], axis=0) * (h0[b].astype(np.float64) if h0 is not None else 0)
            for s in range(t + 1):
                acc = acc + np.prod(a[s + 1: t + 1], axis=0) * inc[s]
            H[b, t] = acc
    y = np.einsum("bldn,bln->bld", H, Cm) + dvec.astype(np.float64) * u
    if z is not None:
        y = y * _silu(z.astype(np.float64).reshape(B, L, D))
    return y.reshape(B * L, D), H


def pin_bruteforce_unrolled(orc):
    B, L, D, N = 2, 12, 3, 4
    inp = _scan_inputs(8, B, L, D, N)
    for disc in (ZOH, EULER):
        y, hc, hl = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                       inp["D_vec"], inp["z"], inp["h0"], batch=B, seq_len=L,
                                       disc=disc, h_cache=True, h_last=True)
        wy, wh = _bruteforce(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                             inp["D_vec"], inp["z"], inp["h0"], B, L, disc)
        _close(hc, wh, 1e-10, 1e-13, f"brute h {disc}")
        _close(hl, wh[:, -1], 1e-10, 1e-13, f"brute h_last {disc}")
        _close(y, wy, 1e-10, 1e-13, f"brute y {disc}")


def pin_core_is_conv_then_scan(orc):
    """core(x) == brute-force scan of u = SiLU(numpy convolve(x))."""
    B, L, D, N, K = 2, 10, 3, 4, 4
    g = _rng(9)
    inp = _scan_inputs(9, B, L, D, N)
    x = _f32(g.standard_normal((B * L, D)))
    w = _f32(0.5 * g.standard_normal((D, K)))
    bias = _f32(0.3 * g.standard_normal(D))
    xs = x.astype(np.float64).reshape(B, L, D)
    c = np.empty((B, L, D))
    for b in range(B):
        for d in range(D):
            c[b, :, d] = np.convolve(xs[b, :, d], w[d].astype(np.float64))[:L] + bias[d]
    u = _silu(c).reshape(B * L, D)
    for disc in (ZOH, EULER):
        y, hc, _ = orc.mamba1_core(x, w, bias, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                   inp["D_vec"], inp["z"], inp["h0"], batch=B, seq_len=L,
                                   disc=disc, h_cache=True)
        wy, wh = _bruteforce(u, inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D_vec"],
                             inp["z"], inp["h0"], B, L, disc)
        _close(hc, wh, 1e-10, 1e-13, f"core h {disc}")
        _close(y, wy, 1e-10, 1e-13, f"core y {disc}")


def pin_hcache_consistent_with_output(orc):
    B, L, D, N = 2, 20, 5, 4
    inp = _scan_inputs(10, B, L, D, N)
    y, hc, _ = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                  inp["D_vec"], inp["z"], None, batch=B, seq_len=L, disc=ZOH,
                                  h_cache=True)
    yy = np.einsum("bldn,bln->bld", hc,
                   inp["C"].astype(np.float64).reshape(B, L, N)).reshape(B * L, D)
    yy = (yy + inp["D_vec"] * inp["u"].astype(np.float64)) * _silu(inp["z"].astype(np.float64))
    _close(y, yy, 1e-12, 1e-14, "hcache vs y")


# --------------------------------------------------------------------------
# invariants


def pin_causality(orc):
    B, L, D, N, K = 2, 40, 6, 4, 4
    g = _rng(11)
    inp = _scan_inputs(11, B, L, D, N)
    x = _f32(g.standard_normal((B * L, D)))
    w = _f32(0.5 * g.standard_normal((D, K)))
    args = lambda xx: (xx, w, None, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                       inp["D_vec"], inp["z"])
    kw = dict(batch=B, seq_len=L, disc=ZOH)
    y0, _, _ = orc.mamba1_core(*args(x), **kw)
    t0 = 20
    x2 = x.copy()
    x2[L + t0] += 1.0  # batch 1, time t0
    y1, _, _ = orc.mamba1_core(*args(x2), **kw)
    y0 = y0.reshape(B, L, D)
    y1 = y1.reshape(B, L, D)
    assert np.array_equal(y0[0], y1[0]), "batch 0 changed"
    assert np.array_equal(y0[1, :t0], y1[1, :t0]), "past of batch 1 changed"
    assert np.all(y0[1, t0] != y1[1, t0]), "perturbed step unchanged"


def pin_alog_clamp_invariance(orc):
    B, L, D, N = 1, 24, 4, 6
    inp = _scan_inputs(12, B, L, D, N)
    base = np.log(np.arange(1, N + 1, dtype=np.float64))[None].repeat(D, 0)
    base[0, 0], base[1, 2] = -12.0, 6.0
    base = _f32(base)

    def run(al):
        y, hc, _ = orc.selective_scan(inp["u"], inp["delta"], _f32(al), inp["B"], inp["C"],
                                      inp["D_vec"], inp["z"], None, batch=B, seq_len=L,
                                      disc=ZOH, h_cache=True)
        return y, hc

    y0, h0 = run(base)
    for lo, hi in ((-30.0, 50.0), (-10.0, 5.0), (-10.5, 5.5)):
        al = base.copy()
        al[0, 0], al[1, 2] = lo, hi
        y1, h1 = run(al)
        assert np.array_equal(y0, y1) and np.array_equal(h0, h1), f"clamp ({lo},{hi}) not invariant"
    for lo, hi in ((-9.5, 6.0), (-12.0, 4.5)):
        al = base.copy()
        al[0, 0], al[1, 2] = lo, hi
        y1, _ = run(al)
        assert not np.array_equal(y0, y1), f"A_log=({lo},{hi}) inside the range had no effect"


def pin_linearity_and_zero_inputs(orc):
    B, L, D, N = 2, 16, 5, 4
    inp = _scan_inputs(13, B, L, D, N)
    kw = dict(batch=B, seq_len=L, disc=ZOH)

    def run(u=inp["u"], Bm=inp["B"], Cm=inp["C"]):
        return orc.selective_scan(u, inp["delta"], inp["A_log"], Bm, Cm, inp["D_vec"], inp["z"],
                                  None, **kw)[0]

    y0 = inp["D_vec"].astype(np.float64) * inp["u"].astype(np.float64) * \
        _silu(inp["z"].astype(np.float64))
    _close(run(Bm=np.zeros_like(inp["B"])), y0, 1e-14, 0.0, "B=0")
    _close(run(Cm=np.zeros_like(inp["C"])), y0, 1e-14, 0.0, "C=0")
    y1 = run()
    _close(run(Bm=2 * inp["B"]) - y0, 2 * (y1 - y0), 1e-12, 1e-13, "linear in B")
    _close(run(Cm=2 * inp["C"]) - y0, 2 * (y1 - y0), 1e-12, 1e-13, "linear in C")
    _close(run(u=2 * inp["u"]), 2 * y1, 1e-12, 1e-13, "linear in u")


def pin_batch_independence(orc):
    B, L, D, N, K = 3, 14, 4, 4, 3
    g = _rng(14)
    inp = _scan_inputs(14, B, L, D, N)
    x = _f32(g.standard_normal((B * L, D)))
    w = _f32(g.standard_normal((D, K)))
    perm = [2, 0, 1]

    def rows(a, width):
        return a.reshape(B, L, width)[perm].reshape(B * L, width)

    y0, hc0, hl0 = orc.mamba1_core(x, w, None, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                   inp["D_vec"], inp["z"], inp["h0"], batch=B, seq_len=L,
                                   disc=EULER, h_cache=True, h_last=True)
    y1, hc1, hl1 = orc.mamba1_core(rows(x, D), w, None, rows(inp["delta"], D), inp["A_log"],
                                   rows(inp["B"], N), rows(inp["C"], N), inp["D_vec"],
                                   rows(inp["z"], D), inp["h0"][perm], batch=B, seq_len=L,
                                   disc=EULER, h_cache=True, h_last=True)
    assert np.array_equal(rows(y0, D), y1)
    assert np.array_equal(hc0[perm], hc1)
    assert np.array_equal(hl0[perm], hl1)


def pin_thread_count_and_columns(orc):
    B, L, D, N, K = 2, 33, 7, 4, 4
    g = _rng(15)
    inp = _scan_inputs(15, B, L, D, N)
    x = _f32(g.standard_normal((B * L, D)))
    w = _f32(g.standard_normal((D, K)))
    args = (x, w, None, inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D_vec"], inp["z"],
            inp["h0"])
    kw = dict(batch=B, seq_len=L, disc=ZOH, h_cache=True, h_last=True)
    r1 = orc.mamba1_core(*args, **kw, nthreads=1)
    r8 = orc.mamba1_core(*args, **kw, nthreads=8)
    for a, b in zip(r1, r8):
        assert np.array_equal(a, b), "thread count changed the result"
    cols = np.array([0, 3, D + 2, 2 * D - 1])
    c = orc.mamba1_core(*args, **kw, cols=cols)
    y = r1[0].reshape(B, L, D)
    for i, col in enumerate(cols):
        b, d = divmod(int(col), D)
        assert np.array_equal(c[0][i], y[b, :, d])
        assert np.array_equal(c[1][i], r1[1][b, :, d])
        assert np.array_equal(c[2][i], r1[2][b, d])


def pin_h0_continues_a_split_sequence(orc):
    B, L, D, N = 2, 30, 4, 4
    inp = _scan_inputs(16, B, L, D, N)
    kw = dict(disc=ZOH, h_last=True)
    yf, _, _ = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                  inp["D_vec"], inp["z"], None, batch=B, seq_len=L, **kw)
    h = 15

    def part(name, s):
        a = inp[name]
        w = a.shape[1]
        return a.reshape(B, L, w)[:, s].reshape(-1, w)

    first, second = slice(0, h), slice(h, L)
    _, _, hl = orc.selective_scan(part("u", first), part("delta", first), inp["A_log"],
                                  part("B", first), part("C", first), inp["D_vec"],
                                  part("z", first), None, batch=B, seq_len=h, **kw)
    y2, _, _ = orc.selective_scan(part("u", second), part("delta", second), inp["A_log"],
                                  part("B", second), part("C", second), inp["D_vec"],
                                  part("z", second), _f32(hl), batch=B, seq_len=L - h, **kw)
    yf = yf.reshape(B, L, D)[:, second].reshape(-1, D)
    _close(y2, yf, 1e-6, 1e-7, "split at h0")


# --------------------------------------------------------------------------
# single-token step


def pin_steps_equal_sequence(orc):
    Bt, L, D, N, K = 2, 20, 5, 4, 4
    g = _rng(17)
    inp = _scan_inputs(17, Bt, L, D, N)
    x = _f32(g.standard_normal((Bt * L, D)))
    w = _f32(0.5 * g.standard_normal((D, K)))
    bias = _f32(0.2 * g.standard_normal(D))
    for disc in (ZOH, EULER):
        y, hc, _ = orc.mamba1_core(x, w, bias, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                   inp["D_vec"], inp["z"], None, batch=Bt, seq_len=L, disc=disc,
                                   h_cache=True)
        y = y.reshape(Bt, L, D)
        cs = np.zeros((Bt, K - 1, D))
        h = np.zeros((Bt, D, N))
        at = lambda a, t, w_: a.reshape(Bt, L, w_)[:, t]
        for t in range(L):
            yt, cs, h = orc.selective_step(at(x, t, D), at(inp["z"], t, D), at(inp["delta"], t, D),
                                           inp["A_log"], at(inp["B"], t, N), at(inp["C"], t, N),
                                           inp["D_vec"], w, bias, cs, h, disc=disc)
            _close(yt, y[:, t], 1e-13, 1e-15, f"step y t={t} {disc}")
            _close(h, hc[:, t], 1e-13, 1e-15, f"step h t={t} {disc}")
            lo = max(0, t - K + 2)
            want_cs = np.zeros((Bt, K - 1, D))
            want_cs[:, K - 1 - (t + 1 - lo):] = x.reshape(Bt, L, D)[:, lo:t + 1]
            assert np.array_equal(cs, want_cs), f"conv state after t={t}"


def pin_step_from_carried_state(orc):
    """A step taken from (last K-1 inputs, h_last) of a prefix continues the sequence."""
    Bt, L, D, N, K = 2, 24, 4, 4, 4
    g = _rng(18)
    inp = _scan_inputs(18, Bt, L, D, N)
    x = _f32(g.standard_normal((Bt * L, D)))
    w = _f32(0.5 * g.standard_normal((D, K)))
    p = 17
    y, _, _ = orc.mamba1_core(x, w, None, inp["delta"], inp["A_log"], inp["B"], inp["C"],
                              inp["D_vec"], inp["z"], None, batch=Bt, seq_len=L, disc=ZOH)
    sl = lambda a, w_, s: a.reshape(Bt, L, w_)[:, s].reshape(-1, w_)
    _, _, hl = orc.mamba1_core(sl(x, D, slice(0, p)), w, None, sl(inp["delta"], D, slice(0, p)),
                               inp["A_log"], sl(inp["B"], N, slice(0, p)),
                               sl(inp["C"], N, slice(0, p)), inp["D_vec"],
                               sl(inp["z"], D, slice(0, p)), None, batch=Bt, seq_len=p,
                               disc=ZOH, h_last=True)
    cs = x.reshape(Bt, L, D)[:, p - K + 1:p].astype(np.float64)
    at = lambda a, t, w_: a.reshape(Bt, L, w_)[:, t]
    yt, _, _ = orc.selective_step(at(x, p, D), at(inp["z"], p, D), at(inp["delta"], p, D),
                                  inp["A_log"], at(inp["B"], p, N), at(inp["C"], p, N),
                                  inp["D_vec"], w, None, cs, hl, disc=ZOH)
    _close(yt, y.reshape(Bt, L, D)[:, p], 1e-13, 1e-15, "step after prefix")


# --------------------------------------------------------------------------
# Backward passes: pinned to central finite differences of the (separately
# pinned) forward oracle, and to a closed form evaluated in 60-digit decimal
# arithmetic.

_BWD_INPUTS = ("u", "delta", "A_log", "B", "C", "D_vec", "z", "h0")
_GRAD_OF = {"u": "du", "delta": "ddelta", "A_log": "dA_log", "B": "dB", "C": "dC",
            "D_vec": "dD", "z": "dz", "h0": "dh0"}


def _fd_element(f, arr, idx, rel=2.0 ** -11):
    """Central difference of f at arr[idx], on the fp32 grid: both perturbed
    values are fp32 numbers and the step is their exact difference."""
    v = float(arr[idx])
    step = rel * max(abs(v), 0.25)
    hi, lo = np.float32(v + step), np.float32(v - step)
    arr[idx] = hi
    fp = f()
    arr[idx] = lo
    fm = f()
    arr[idx] = np.float32(v)
    return (fp - fm) / (float(hi) - float(lo))


def _scan_loss(orc, inp, dout, B, L, disc):
    def f():
        y, _, _ = orc.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                     inp["D_vec"], inp["z"], inp["h0"], batch=B, seq_len=L,
                                     disc=disc)
        return float(np.sum(y * dout))
    return f


def _check_scan_grads(orc, inp, dout, B, L, disc, picks=None, rtol=2e-5):
    g = orc.selective_scan_backward(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                    inp["D_vec"], inp["z"], inp["h0"], dout, batch=B,
                                    seq_len=L, disc=disc)
    f = _scan_loss(orc, inp, dout, B, L, disc)
    rs = _rng(99)
    for name in _BWD_INPUTS:
        arr = inp[name]
        grad = g[_GRAD_OF[name]].reshape(arr.shape)
        scale = float(np.sqrt(np.mean(grad ** 2))) + 1e-30
        idxs = list(np.ndindex(arr.shape))
        if picks is not None and len(idxs) > picks:
            idxs = [idxs[i] for i in rs.choice(len(idxs), picks, replace=False)]
        for idx in idxs:
            fd = _fd_element(f, arr, idx)
            assert abs(fd - grad[idx]) <= rtol * (abs(grad[idx]) + scale), (
                f"{disc} d/d{name}{idx}: oracle {grad[idx]:.10e} vs finite difference {fd:.10e}")


def pin_scan_backward_finite_differences(orc):
    # Every element of every input, both modes; A_log has entries on both
    # sides of the clamp (their gradient must be exactly zero).
    B, L, D, N = 2, 6, 3, 4
    for disc in (ZOH, EULER):
        inp = _scan_inputs(31, B, L, D, N, alog_lo=-2.0, alog_hi=1.5)
        inp["A_log"][0, 1] = -11.5
        inp["A_log"][2, 3] = 5.75
        dout = _f32(_rng(32).standard_normal((B * L, D)))
        _check_scan_grads(orc, inp, dout, B, L, disc)
        g = orc.selective_scan_backward(inp["u"], inp["delta"], inp["A_log"], inp["B"],
                                        inp["C"], inp["D_vec"], inp["z"], inp["h0"], dout,
                                        batch=B, seq_len=L, disc=disc)
        assert g["dA_log"][0, 1] == 0.0 and g["dA_log"][2, 3] == 0.0


def pin_scan_backward_long_memory(orc):
    # Slow decay (small dv, small |A|), so gradients of early steps travel
    # through the carried adjoint across the whole sequence; no gate, no h0.
    B, L, D, N = 1, 48, 2, 3
    for disc in (ZOH, EULER):
        inp = _scan_inputs(41, B, L, D, N, alog_lo=-3.0, alog_hi=-1.0, delta_mu=-2.0)
        inp["z"] = None
        inp["h0"] = None
        dout = _f32(_rng(42).standard_normal((B * L, D)))
        g = orc.selective_scan_backward(inp["u"], inp["delta"], inp["A_log"], inp["B"],
                                        inp["C"], inp["D_vec"], None, None, dout, batch=B,
                                        seq_len=L, disc=disc)
        assert g["dz"] is None
        f = _scan_loss(orc, inp, dout, B, L, disc)
        for name, idx in (("u", (0, 0)), ("u", (3, 1)), ("delta", (1, 0)), ("delta", (2, 1)),
                          ("B", (0, 2)), ("B", (1, 0)), ("A_log", (0, 0)), ("A_log", (1, 2)),
                          ("C", (47, 1)), ("D_vec", (1,))):
            arr = inp[name]
            grad = g[_GRAD_OF[name]].reshape(arr.shape)
            fd = _fd_element(f, arr, idx)
            assert abs(fd - grad[idx]) <= 2e-5 * (abs(grad[idx]) + 1e-3), (
                f"{disc} long d/d{name}{idx}: {grad[idx]:.10e} vs {fd:.10e}")


def pin_scan_backward_thread_count(orc):
    # The cross-channel sums run in a fixed order: any thread count gives
    # bitwise the same gradients (D = 150 spans three channel blocks).
    B, L, D, N = 2, 40, 150, 4
    inp = _scan_inputs(71, B, L, D, N)
    dout = _f32(_rng(72).standard_normal((B * L, D)))
    args = (inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D_vec"], inp["z"],
            inp["h0"], dout)
    g1 = orc.selective_scan_backward(*args, batch=B, seq_len=L, disc=ZOH, nthreads=1)
    g5 = orc.selective_scan_backward(*args, batch=B, seq_len=L, disc=ZOH, nthreads=5)
    for k in g1:
        assert np.array_equal(g1[k], g5[k]), k


def pin_zoh_a_grad_tiny_step_closed_form(orc):
    # L = 1, h0 = 0, one state, ungated, no skip: y = C u B expm1(dv A) / A,
    # so dy/dA_log = C u B (x e^x - expm1(x)) / A with x = dv A, A = -e^A_log.
    # Evaluated in 60-digit decimal arithmetic, for |x| from 1e-9 to 1.
    import decimal
    ctx = decimal.Context(prec=60)
    Dm = decimal.Decimal
    for delta, alog in ((-20.0, 0.3), (-9.0, -1.0), (-4.0, 0.5), (0.5, 0.0), (-1.0, 1.2)):
        u = _f32([[1.25]])
        dl = _f32([[delta]])
        al = _f32([[alog]])
        Bm, Cm = _f32([[0.75]]), _f32([[-1.5]])
        dout = _f32([[1.0]])
        g = orc.selective_scan_backward(u, dl, al, Bm, Cm, None, None, None, dout, batch=1,
                                        seq_len=1, disc=ZOH)
        dd = Dm(float(dl[0, 0]))
        dv = ctx.add(max(dd, Dm(0)), ctx.ln(ctx.add(Dm(1), ctx.exp(-abs(dd)))))
        A = -ctx.exp(Dm(float(al[0, 0])))
        x = ctx.multiply(dv, A)
        em1 = ctx.subtract(ctx.exp(x), Dm(1))
        want = (Dm(float(Cm[0, 0])) * Dm(float(u[0, 0])) * Dm(float(Bm[0, 0])) *
                ctx.divide(ctx.subtract(ctx.multiply(x, ctx.exp(x)), em1), A))
        got = g["dA_log"][0, 0]
        assert abs(Dm(got) - want) <= abs(want) * Dm("1e-12"), (
            f"delta={delta}: {got!r} vs {want}")


def pin_conv_backward_finite_differences(orc):
    Bt, L, D, K = 2, 7, 3, 4
    g = _rng(51)
    x = _f32(g.standard_normal((Bt * L, D)))
    w = _f32(0.5 * g.standard_normal((D, K)))
    b = _f32(0.3 * g.standard_normal(D))
    du = _f32(g.standard_normal((Bt * L, D)))
    dx, dw, db = orc.conv1d_silu_backward(x, w, b, du, batch=Bt, seq_len=L)

    def f():
        return float(np.sum(orc.conv1d_silu(x, w, b, batch=Bt, seq_len=L) * du))
    for arr, grad, nm in ((x, dx, "x"), (w, dw, "w"), (b, db, "b")):
        scale = float(np.sqrt(np.mean(grad ** 2)))
        for idx in np.ndindex(arr.shape):
            fd = _fd_element(f, arr, idx)
            assert abs(fd - grad[idx]) <= 2e-5 * (abs(grad[idx]) + scale), (
                f"conv d/d{nm}{idx}: oracle {grad[idx]:.10e} vs finite difference {fd:.10e}")


# --------------------------------------------------------------------------
# Mamba-2 SSD scan


def _ssd_inputs(seed, B, L, H, P, N, G, *, h0=True, bias=True):
    g = _rng(seed)
    return dict(
        x=_f32(g.standard_normal((B * L, H * P))),
        dt=_f32(g.standard_normal((B * L, H)) - 1.0),
        A_log=_f32(g.uniform(-1.0, 2.5, H)),
        B=_f32(g.standard_normal((B * L, G * N))),
        C=_f32(g.standard_normal((B * L, G * N))),
        D_vec=_f32(g.uniform(0.5, 1.5, H)),
        dt_bias=_f32(g.uniform(-0.5, 0.5, H)) if bias else None,
        h0=_f32(0.3 * g.standard_normal((B, H, P, N))) if h0 else None,
    )


def _ssd(orc, inp, B, L, H, P, N, G, disc=EULER, **kw):
    return orc.ssd_scan(inp["x"], inp["dt"], inp["A_log"], inp["B"], inp["C"], inp["D_vec"],
                        inp["dt_bias"], inp["h0"], batch=B, seq_len=L, n_heads=H, head_dim=P,
                        d_state=N, n_groups=G, disc=disc, h_last=True, **kw)


def pin_ssd_is_mamba1_per_channel(orc):
    # Channel (h, p) of the SSD scan is the Mamba-1 scan (same discretisation)
    # of one channel whose N states all have A_h, on delta = dt + dt_bias,
    # with the B and C of the head's group: run the (separately pinned)
    # Mamba-1 oracle group by group and compare y and the final state.
    for disc in (EULER, ZOH):
        _ssd_vs_mamba1(orc, disc)


def _ssd_vs_mamba1(orc, disc):
    B, L, H, P, N, G = 2, 23, 6, 3, 5, 3
    inp = _ssd_inputs(61, B, L, H, P, N, G)
    y, hl = _ssd(orc, inp, B, L, H, P, N, G, disc=disc)
    hpg = H // G
    for g in range(G):
        heads = range(g * hpg, (g + 1) * hpg)
        cols = [h * P + p for h in heads for p in range(P)]
        delta = np.concatenate([np.repeat((inp["dt"][:, h].astype(np.float64) +
                                           inp["dt_bias"][h])[:, None], P, axis=1)
                                for h in heads], axis=1)
        # delta is rounded to fp32 on the way into the Mamba-1 oracle; keep
        # only inputs where that is exact by comparing with a tolerance
        alog = np.repeat(np.repeat(inp["A_log"][list(heads)], P)[:, None], N, axis=1)
        y1, _, hl1 = orc.selective_scan(
            inp["x"][:, cols], _f32(delta), _f32(alog), inp["B"][:, g * N:(g + 1) * N],
            inp["C"][:, g * N:(g + 1) * N], np.repeat(inp["D_vec"][list(heads)], P), None,
            inp["h0"][:, list(heads)].reshape(B, hpg * P, N), batch=B, seq_len=L,
            disc=disc, h_last=True)
        _close(y[:, cols], y1, 1e-6, 1e-6, f"ssd vs mamba1, group {g}")
        _close(hl[:, list(heads)].reshape(B, hpg * P, N), hl1, 1e-6, 1e-6,
               f"ssd h_last vs mamba1, group {g}")


def pin_ssd_exact_shift_of_dt(orc):
    # With dt and dt_bias on a coarse dyadic grid, dt + dt_bias is exact in
    # fp32, so adding the bias inside equals adding it outside, bitwise.
    B, L, H, P, N, G = 1, 17, 4, 2, 3, 2
    inp = _ssd_inputs(62, B, L, H, P, N, G)
    inp["dt"] = _f32(np.round(inp["dt"] * 64) / 64)
    inp["dt_bias"] = _f32(np.round(inp["dt_bias"] * 64) / 64)
    for disc in (EULER, ZOH):
        y, hl = _ssd(orc, inp, B, L, H, P, N, G, disc=disc)
        moved = dict(inp, dt=_f32(inp["dt"] + inp["dt_bias"][None, :]), dt_bias=None)
        y2, hl2 = _ssd(orc, moved, B, L, H, P, N, G, disc=disc)
        assert np.array_equal(y, y2) and np.array_equal(hl, hl2)


def pin_ssd_quadratic_form(orc):
    # The scan equals its unrolled (attention-like) form, evaluated here
    # directly in fp64 for every output:
    #   y[t,h,p] = sum_{s<=t} (C_t . B_s) exp(A_h sum_{r=s+1..t} dv_r) f_s x[s,h,p]
    #              + sum_n C_t,n exp(A_h sum_{r<=t} dv_r) h0[h,p,n] + D_h x[t,h,p]
    # with f = dv (EULER), checked here; ZOH's f is pinned by the Mamba-1 pin.
    B, L, H, P, N, G = 2, 12, 4, 3, 4, 2
    inp = _ssd_inputs(63, B, L, H, P, N, G)
    y, hl = _ssd(orc, inp, B, L, H, P, N, G)
    hpg = H // G
    want = np.zeros((B * L, H * P))
    for b in range(B):
        for h in range(H):
            g = h // hpg
            A = -np.exp(np.clip(np.float64(inp["A_log"][h]), -10.0, 5.0))
            dv = _softplus(inp["dt"][b * L:(b + 1) * L, h].astype(np.float64) + inp["dt_bias"][h])
            cum = np.concatenate([[0.0], np.cumsum(dv)])      # cum[t+1] = sum_{r<=t} dv_r
            Bg = inp["B"][b * L:(b + 1) * L, g * N:(g + 1) * N].astype(np.float64)
            Cg = inp["C"][b * L:(b + 1) * L, g * N:(g + 1) * N].astype(np.float64)
            xs = inp["x"][b * L:(b + 1) * L, h * P:(h + 1) * P].astype(np.float64)
            for t in range(L):
                acc = inp["D_vec"][h] * xs[t]
                for s_ in range(t + 1):
                    acc = acc + (Cg[t] @ Bg[s_]) * np.exp(A * (cum[t + 1] - cum[s_ + 1])) * dv[s_] * xs[s_]
                acc = acc + np.exp(A * cum[t + 1]) * (inp["h0"][b, h].astype(np.float64) @ Cg[t])
                want[b * L + t, h * P:(h + 1) * P] = acc
    _close(y, want, 1e-12, 1e-12, "ssd quadratic form")


def pin_ssd_clamp_and_groups(orc):
    # A_log beyond the clamp: same output bitwise; heads of one group with
    # identical inputs give identical outputs; groups do not leak.
    B, L, H, P, N, G = 1, 15, 4, 2, 3, 2
    inp = _ssd_inputs(64, B, L, H, P, N, G)
    inp["A_log"][0] = -10.0
    inp["A_log"][1] = 5.0
    y, _ = _ssd(orc, inp, B, L, H, P, N, G)
    far = dict(inp, A_log=inp["A_log"].copy())
    far["A_log"][0] = -30.0
    far["A_log"][1] = 40.0
    y2, _ = _ssd(orc, far, B, L, H, P, N, G)
    assert np.array_equal(y, y2)
    same = dict(inp)
    for k_ in ("x",):
        a = inp[k_].copy()
        a[:, P:2 * P] = a[:, 0:P]
        same[k_] = a
    for k_ in ("dt",):
        a = inp[k_].copy()
        a[:, 1] = a[:, 0]
        same[k_] = a
    for k_ in ("A_log", "D_vec", "dt_bias"):
        a = inp[k_].copy()
        a[1] = a[0]
        same[k_] = a
    same["h0"] = inp["h0"].copy()
    same["h0"][:, 1] = same["h0"][:, 0]
    y3, _ = _ssd(orc, same, B, L, H, P, N, G)
    assert np.array_equal(y3[:, 0:P], y3[:, P:2 * P])
    other = dict(same, B=same["B"].copy())
    other["B"][:, N:] += 1.0          # group 1 only: heads 2, 3
    y4, _ = _ssd(orc, other, B, L, H, P, N, G)
    assert np.array_equal(y4[:, :2 * P], y3[:, :2 * P])
    assert not np.allclose(y4[:, 2 * P:], y3[:, 2 * P:])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
