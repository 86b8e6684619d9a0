"""State checkpoints every 8 steps (MSS_FLAG_CKPT8), on the GPU.

A forward call with the flag writes, instead of every step's state, the
state entering steps 0, 8, 16, ... (entry k = h_{8k-1}, entry 0 = h0 or 0);
the scan backward given those checkpoints starts each 8-step block from
them instead of rebuilding the forward states itself.  Checked against the
fp64 oracle: the checkpoints against the oracle's state cache at steps
8k - 1, every gradient of the backward against the oracle's, and the
allocation-free backward bit for bit against the workspace one."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import mamba_selective_scan_causal_amd as mss
from mamba_selective_scan_causal_amd import inputs as gen
from gpu_util import announce, assert_close, dev, host, nan_like

pytestmark = pytest.mark.gpu

DISCS = ("zoh", "euler")
GRADS = ("du", "ddelta", "dA_log", "dB", "dC", "dD", "dz", "dh0")


@pytest.fixture(autouse=True)
def _announce(request):
    announce(request.node.nodeid)
    yield


def _inputs(w):
    inp = gen.generate(w)
    inp["u"] = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=w.batch,
                                  seq_len=w.seq_len).astype(np.float32)
    inp["dout"] = gen.cotangent(w)
    return inp


def _oracle_ckpt(hc, h0, w):
    """(B, ceil(L/8), D, N) from the oracle's (B, L, D, N) state cache."""
    B, L, D, N = w.batch, w.seq_len, w.d_inner, w.d_state
    out = np.empty((B, (L + 7) // 8, D, N))
    out[:, 0] = h0 if h0 is not None else 0.0
    for k in range(1, (L + 7) // 8):
        out[:, k] = hc[:, 8 * k - 1]
    return out


def _gpu_ckpt(d, w, disc, *, fused, exact=False):
    import torch
    B, L, D, N = w.batch, w.seq_len, w.d_inner, w.d_state
    ck = nan_like((B, mss.ckpt_steps(L), D, N))
    y = nan_like((B * L, D))
    if fused:
        mss.mamba1_core(d["x"], d["w_conv"], d["b_conv"], d["delta"], d["A_log"], d["B"], d["C"],
                        d["D_vec"], d["z"], d.get("h0"), batch=B, seq_len=L, disc=disc,
                        h_cache=ck, ckpt8=True, out=y, exact=exact)
    else:
        mss.selective_scan(d["u"], d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"], d["z"],
                           d.get("h0"), batch=B, seq_len=L, disc=disc, h_cache=ck, ckpt8=True,
                           out=y, exact=exact)
    torch.cuda.synchronize()
    return ck, y


CK_CASES = [
    gen.TINY_CLAMP,
    gen.SMALL.with_(h0=True),
    gen.SMALL.with_(name="ragged", batch=2, seq_len=203, d_inner=70, h0=True),
    gen.SMALL.with_(name="len9", batch=3, seq_len=9, d_inner=64, h0=True),
    gen.SMALL.with_(name="len1", batch=2, seq_len=1, d_inner=33),
    gen.SMALL.with_(name="n5", batch=2, seq_len=300, d_inner=40, d_state=5, h0=True),
    gen.SMALL.with_(name="k3", batch=2, seq_len=301, d_inner=96, d_conv=3, h0=True),
    gen.MAMBA_130M,
]


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("fused", (True, False), ids=("core", "scan"))
@pytest.mark.parametrize("w", CK_CASES, ids=lambda w: w.name)
def test_forward_checkpoints(w, fused, disc):
    inp = _inputs(w)
    d = {k: dev(v) for k, v in inp.items()}
    ck, y = _gpu_ckpt(d, w, disc, fused=fused)
    if fused:
        oy, ohc, _ = oracle.mamba1_core(inp["x"], inp["w_conv"], inp["b_conv"], inp["delta"],
                                        inp["A_log"], inp["B"], inp["C"], inp["D_vec"], inp["z"],
                                        inp.get("h0"), batch=w.batch, seq_len=w.seq_len,
                                        disc=disc, h_cache=True)
    else:
        oy, ohc, _ = oracle.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"],
                                           inp["C"], inp["D_vec"], inp["z"], inp.get("h0"),
                                           batch=w.batch, seq_len=w.seq_len, disc=disc,
                                           h_cache=True)
    assert_close(host(y), oy, "y")
    assert_close(host(ck), _oracle_ckpt(ohc, inp.get("h0"), w), "checkpoints")


def _bwd(d, w, disc, ck=None, noalloc=False):
    import torch
    f = mss.selective_scan_backward_noalloc if noalloc else mss.selective_scan_backward
    g = f(d["u"], d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"], d["z"], d.get("h0"),
          d["dout"], batch=w.batch, seq_len=w.seq_len, disc=disc, need_dh0=True, h_ckpt=ck)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in g.items()}


def _check(got, want, what):
    errs = {k: assert_close(got[k], want[k], f"{what}: {k}") for k in GRADS}
    announce(what + " " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))


BWD_CASES = CK_CASES + [
    gen.SMALL.with_(name="slow_decay", batch=1, seq_len=1500, d_inner=64, alog_clamp_frac=1.0,
                    h0=True),
    gen.SMALL.with_(name="tiny_steps", batch=2, seq_len=1200, d_inner=64, delta_mean=-9.0,
                    delta_var=1.0, h0=True),
]


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: w.name)
def test_backward_from_checkpoints(w, disc):
    inp = _inputs(w)
    d = {k: dev(v) for k, v in inp.items()}
    ck, _ = _gpu_ckpt(d, w, disc, fused=False)
    got = _bwd(d, w, disc, ck)
    want = oracle.selective_scan_backward(inp["u"], inp["delta"], inp["A_log"], inp["B"],
                                          inp["C"], inp["D_vec"], inp["z"], inp.get("h0"),
                                          inp["dout"], batch=w.batch, seq_len=w.seq_len,
                                          disc=disc)
    _check(got, want, "from checkpoints")
    # the allocation-free entry point takes the same checkpoints, bit for bit
    na = _bwd(d, w, disc, ck, noalloc=True)
    for k in GRADS:
        assert np.array_equal(na[k], got[k]), k


@pytest.mark.parametrize("disc", DISCS)
def test_backward_from_checkpoints_full_size(disc):
    """B4 L8192 D5120 N16, gated: the forward writes its checkpoints, the
    backward starts from them; every gradient against the oracle on the
    whole problem."""
    w = gen.MAMBA_2P8B
    inp = _inputs(w)
    d = {k: dev(v) for k, v in inp.items()}
    ck, _ = _gpu_ckpt(d, w, disc, fused=False)
    got = _bwd(d, w, disc, ck)
    want = oracle.selective_scan_backward(inp["u"], inp["delta"], inp["A_log"], inp["B"],
                                          inp["C"], inp["D_vec"], inp["z"], None, inp["dout"],
                                          batch=w.batch, seq_len=w.seq_len, disc=disc)
    _check(got, want, "full size from checkpoints")


@pytest.mark.parametrize("disc", DISCS)
def test_exact_forward_checkpoints_feed_exact_backward(disc):
    """MSS_FLAG_EXACT on both sides, with an outlier of 1e6 in u: the
    checkpoints and the backward match the oracle."""
    w = gen.SMALL.with_(name="exact_ck", batch=2, seq_len=1500, d_inner=96, h0=True)
    inp = _inputs(w)
    inp["u"][700, :] = 1e6
    d = {k: dev(v) for k, v in inp.items()}
    ck, _ = _gpu_ckpt(d, w, disc, fused=False, exact=True)
    _, ohc, _ = oracle.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                      inp["D_vec"], inp["z"], inp["h0"], batch=w.batch,
                                      seq_len=w.seq_len, disc=disc, h_cache=True)
    assert_close(host(ck), _oracle_ckpt(ohc, inp["h0"], w), "checkpoints")
    import torch
    g = mss.selective_scan_backward(d["u"], d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"],
                                    d["z"], d["h0"], d["dout"], batch=w.batch, seq_len=w.seq_len,
                                    disc=disc, need_dh0=True, h_ckpt=ck, exact=True)
    torch.cuda.synchronize()
    want = oracle.selective_scan_backward(inp["u"], inp["delta"], inp["A_log"], inp["B"],
                                          inp["C"], inp["D_vec"], inp["z"], inp["h0"],
                                          inp["dout"], batch=w.batch, seq_len=w.seq_len,
                                          disc=disc)
    _check({k: host(v) for k, v in g.items()}, want, "exact")


@pytest.mark.parametrize("disc", DISCS)
@pytest.mark.parametrize("entry", ("core", "scan"))
def test_strided_forward_checkpoints(entry, disc):
    """The strided entry points with MSS_FLAG_CKPT8: x, z as the halves of an
    (M, 2D) buffer, B, C as an unaligned column range of an (M, R + 2N) one,
    delta and y as column slices; the checkpoints match the oracle's state
    cache, nothing outside y's slice is written, and the backward started
    from them matches the oracle's gradients."""
    import torch
    w = gen.SMALL.with_(name="strided_ck", batch=2, seq_len=1203, d_inner=160, h0=True)
    inp = _inputs(w)
    M, D, N, B, L, R = w.M, w.d_inner, w.d_state, w.batch, w.seq_len, 5
    g = np.random.default_rng(16)
    junk = lambda c: g.standard_normal((M, c)).astype(np.float32)
    src = inp["x"] if entry == "core" else inp["u"]
    XZ = dev(np.concatenate([src, inp["z"]], axis=1))
    XP = dev(np.concatenate([junk(R), inp["B"], inp["C"]], axis=1))
    DP = dev(np.concatenate([inp["delta"], junk(3)], axis=1))
    YB = nan_like((M, D + 7))
    x, z = XZ[:, :D], XZ[:, D:]
    Bv, Cv = XP[:, R:R + N], XP[:, R + N:]
    dl, y = DP[:, :D], YB[:, 3:3 + D]
    ck = nan_like((B, mss.ckpt_steps(L), D, N))
    d = {k: dev(inp[k]) for k in ("w_conv", "b_conv", "A_log", "D_vec", "h0")}
    if entry == "core":
        mss.mamba1_core(x, d["w_conv"], d["b_conv"], dl, d["A_log"], Bv, Cv, d["D_vec"], z,
                        d["h0"], batch=B, seq_len=L, disc=disc, h_cache=ck, ckpt8=True, out=y)
    else:
        mss.selective_scan(x, dl, d["A_log"], Bv, Cv, d["D_vec"], z, d["h0"], batch=B,
                           seq_len=L, disc=disc, h_cache=ck, ckpt8=True, out=y)
    torch.cuda.synchronize()
    oy, ohc, _ = oracle.selective_scan(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"],
                                       inp["D_vec"], inp["z"], inp["h0"], batch=B, seq_len=L,
                                       disc=disc, h_cache=True)
    assert_close(host(y), oy, "y")
    assert_close(host(ck), _oracle_ckpt(ohc, inp["h0"], w), "checkpoints")
    outside = torch.cat([YB[:, :3], YB[:, 3 + D:]], dim=1)
    assert torch.isnan(outside).all().item(), "wrote outside the y slice"
    dd = {k: dev(v) for k, v in inp.items()}
    got = _bwd(dd, w, disc, ck)
    want = oracle.selective_scan_backward(inp["u"], inp["delta"], inp["A_log"], inp["B"],
                                          inp["C"], inp["D_vec"], inp["z"], inp["h0"],
                                          inp["dout"], batch=B, seq_len=L, disc=disc)
    _check(got, want, "strided checkpoints")
