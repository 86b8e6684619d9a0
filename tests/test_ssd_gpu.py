"""GPU parity of the Mamba-2 SSD scan (mss_ssd_scan, matrix-core chunked
form) against the fp64 oracle's plain recurrence on the same seeded inputs,
within max relative error 1e-4 (gpu_util.rel_err).  Outputs start as NaN."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import mamba_selective_scan_causal_amd as mss
from mamba_selective_scan_causal_amd import inputs as gen
from gpu_util import announce, assert_close, dev, host, nan_like

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    announce(request.node.nodeid)
    yield


def run_ssd(inp, w, *, disc="euler", dvec=True, bias=True, h0=True):
    import torch
    d = {k: dev(v) for k, v in inp.items()}
    y = nan_like((w.M, w.n_heads * w.head_dim))
    hl = nan_like((w.batch, w.n_heads, w.head_dim, w.d_state))
    mss.ssd_scan(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D_vec"] if dvec else None,
                 d["dt_bias"] if bias else None, d["h0"] if (h0 and "h0" in d) else None,
                 batch=w.batch, seq_len=w.seq_len, head_dim=w.head_dim, d_state=w.d_state,
                 n_groups=w.n_groups, disc=disc, h_last=hl, out=y)
    torch.cuda.synchronize()
    return host(y), host(hl)


def oracle_ssd(inp, w, *, disc="euler", dvec=True, bias=True, h0=True):
    return oracle.ssd_scan(inp["x"], inp["dt"], inp["A_log"], inp["B"], inp["C"],
                           inp["D_vec"] if dvec else None, inp["dt_bias"] if bias else None,
                           inp.get("h0") if h0 else None, batch=w.batch, seq_len=w.seq_len,
                           n_heads=w.n_heads, head_dim=w.head_dim, d_state=w.d_state,
                           n_groups=w.n_groups, disc=disc, h_last=True)


def check(w, inp=None, **kw):
    inp = inp if inp is not None else gen.generate_ssd(w)
    y, hl = run_ssd(inp, w, **kw)
    oy, ohl = oracle_ssd(inp, w, **kw)
    e1 = assert_close(y, oy, "y")
    e2 = assert_close(hl, ohl, "h_last")
    announce(f"errors y={e1:.1e} h_last={e2:.1e}")


@pytest.mark.parametrize("disc", ("euler", "zoh"))
@pytest.mark.parametrize("w", [gen.SSD_TINY, gen.SSD_SMALL], ids=lambda w: w.name)
def test_ssd_workloads(w, disc):
    check(w, disc=disc)


SSD_EDGE = [
    ("ragged_len", dict(batch=2, seq_len=77, n_heads=4, head_dim=64, d_state=128)),
    ("many_segments", dict(batch=1, seq_len=4096, n_heads=2, head_dim=64, d_state=128)),
    ("segments_ragged", dict(batch=2, seq_len=2500, n_heads=3, head_dim=32, d_state=64)),
    ("p128_n128", dict(batch=1, seq_len=300, n_heads=2, head_dim=128, d_state=128)),
    ("p16_n16", dict(batch=2, seq_len=200, n_heads=4, head_dim=16, d_state=16)),
    ("p32_n32_g4", dict(batch=1, seq_len=300, n_heads=8, head_dim=32, d_state=32, n_groups=4)),
    ("p128_n64_g2", dict(batch=1, seq_len=200, n_heads=4, head_dim=128, d_state=64, n_groups=2)),
    ("len1", dict(batch=3, seq_len=1, n_heads=2, head_dim=64, d_state=128)),
    ("len33", dict(batch=1, seq_len=33, n_heads=2, head_dim=64, d_state=32)),
    ("tiny_steps", dict(batch=1, seq_len=1500, n_heads=2, head_dim=64, d_state=64,
                        dt_mean=-9.0, dt_var=1.0)),
]


@pytest.mark.parametrize("name,over", SSD_EDGE, ids=[e[0] for e in SSD_EDGE])
def test_ssd_edge_cases(name, over):
    check(gen.SSD_SMALL.with_(**over))
    if name in ("ragged_len", "many_segments", "tiny_steps"):
        check(gen.SSD_SMALL.with_(**over), disc="zoh")


def test_ssd_no_skip_no_bias_no_h0_and_dt_bias():
    w = gen.SSD_SMALL.with_(batch=1, seq_len=700, n_heads=4)
    check(w, dvec=False, bias=False, h0=False)
    inp = gen.generate_ssd(w)
    inp["dt_bias"] = np.linspace(-1.0, 1.0, w.n_heads).astype(np.float32)
    check(w, inp=inp)


def test_ssd_slow_decay_full_replay():
    """A_log at the lower clamp (A = -4.5e-5): nothing decays, so every
    segment replays from t = 0; the result stays the plain recurrence."""
    w = gen.SSD_SMALL.with_(batch=1, seq_len=3000, n_heads=2, head_dim=32, d_state=32)
    inp = gen.generate_ssd(w)
    inp["A_log"] = np.array([-12.0, 0.5], dtype=np.float32)
    check(w, inp=inp)
    check(w, inp=inp, disc="zoh")


def test_ssd_empty_and_deterministic():
    import torch
    w = gen.SSD_SMALL.with_(batch=2, seq_len=0, n_heads=2)
    inp = gen.generate_ssd(w)
    d = {k: dev(v) for k, v in inp.items()}
    x = torch.empty((0, 2 * 64), device="cuda")
    dt = torch.empty((0, 2), device="cuda")
    bc = torch.empty((0, 128), device="cuda")
    y, hl = mss.ssd_scan(x, dt, d["A_log"], bc, bc, d["D_vec"], None, d["h0"], batch=2,
                         seq_len=0, head_dim=64, d_state=128, disc="euler", h_last=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(hl), inp["h0"].astype(np.float64))
    w = gen.SSD_SMALL.with_(batch=1, seq_len=1000, n_heads=3)
    inp = gen.generate_ssd(w)
    a = run_ssd(inp, w)
    b = run_ssd(inp, w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_ssd_full_size_sampled_heads():
    """B4 L8192 H80 P64 N128 in the benchmark's launch configuration; the
    oracle runs the same inputs restricted to 3 heads (heads of one group
    are independent given B and C)."""
    w = gen.SSD_2P7B
    inp = gen.generate_ssd(w)
    y, hl = run_ssd(inp, w)
    heads = [0, 37, 79]
    P = w.head_dim
    cols = np.concatenate([np.arange(h * P, (h + 1) * P) for h in heads])
    sub = dict(x=inp["x"][:, cols].copy(), dt=inp["dt"][:, heads].copy(),
               A_log=inp["A_log"][heads], B=inp["B"], C=inp["C"], D_vec=inp["D_vec"][heads],
               dt_bias=inp["dt_bias"][heads])
    ws = w.with_(n_heads=len(heads))
    oy, ohl = oracle_ssd(sub, ws, h0=False)
    # the same launch configuration in the other discretisation
    y2, hl2 = run_ssd(inp, w, disc="zoh")
    oy2, ohl2 = oracle_ssd(sub, ws, disc="zoh", h0=False)
    assert_close(y2[:, cols], oy2, "y (zoh)")
    assert_close(hl2[:, heads], ohl2, "h_last (zoh)")
    assert_close(y[:, cols], oy, "y")
    assert_close(hl[:, heads], ohl, "h_last")


GUARD_CASES = [
    ("l100_p16_n32_g2", dict(batch=1, seq_len=100, n_heads=4, head_dim=16, d_state=32, n_groups=2)),
    ("l77_p64_n128", dict(batch=2, seq_len=77, n_heads=4, head_dim=64, d_state=128)),
    ("l33_p128_n64", dict(batch=1, seq_len=33, n_heads=2, head_dim=128, d_state=64)),
    ("l1_p32_n16", dict(batch=3, seq_len=1, n_heads=2, head_dim=32, d_state=16)),
]


@pytest.mark.parametrize("name,over", GUARD_CASES, ids=[c[0] for c in GUARD_CASES])
def test_ssd_writes_nothing_past_its_output(name, over):
    """y is the first M rows of a NaN-filled buffer 64 rows longer: the
    rows past the last chunk's end (a partial chunk here) are never written,
    and y itself matches the oracle."""
    import torch
    w = gen.SSD_SMALL.with_(**over)
    inp = gen.generate_ssd(w)
    d = {k: dev(v) for k, v in inp.items()}
    HP = w.n_heads * w.head_dim
    buf = nan_like((w.M + 64, HP))
    y = buf[:w.M]
    mss.ssd_scan(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D_vec"], d["dt_bias"],
                 d.get("h0"), batch=w.batch, seq_len=w.seq_len, head_dim=w.head_dim,
                 d_state=w.d_state, n_groups=w.n_groups, disc="euler", out=y)
    torch.cuda.synchronize()
    tail = host(buf[w.M:])
    assert np.isnan(tail).all(), f"{int((~np.isnan(tail)).sum())} guard values written"
    oy, _ = oracle_ssd(inp, w)
    assert_close(host(y), oy, "y")


PN = [(p, n) for p in (16, 32, 64, 128) for n in (16, 32, 64, 128)]


@pytest.mark.parametrize("P,N", PN, ids=[f"p{p}_n{n}" for p, n in PN])
def test_ssd_every_head_dim_and_state_size(P, N):
    """Every (P, N) instantiation -- each has its own split of the C B^T
    tiles over the waves and its own register budget -- on 150 steps (time
    segments with replays, a ragged last chunk), h0 and h_last, both
    discretisations across the set."""
    i = PN.index((P, N))
    G = 2 if i % 3 == 0 else 1
    w = gen.SSD_SMALL.with_(name=f"pn_{P}_{N}", batch=1 + i % 2, seq_len=150, n_heads=2 * G,
                            head_dim=P, d_state=N, n_groups=G, h0=True, seed_index=300 + i)
    check(w, disc="zoh" if i % 2 == 0 else "euler")
