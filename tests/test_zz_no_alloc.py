"""The allocation-free scan backward (mss_selective_scan_backward_noalloc,
workspace in the library's static scratch array) against the entry point
with a caller workspace, through the C ABI.

Two calls in a row on the scratch array, the second with a smaller problem
(so it runs on what the first left behind), each compared with the
workspace entry point on the same inputs: the two run the same kernels with
the same split, so the results must agree bit for bit (and so within the
1e-4 of the parity tests).  A third call, larger again, follows a call of
the workspace entry point."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import mamba_selective_scan_causal_amd as mss
from mamba_selective_scan_causal_amd import inputs as gen
from gpu_util import announce, assert_close, dev, host

pytestmark = pytest.mark.gpu

KEYS = ("du", "ddelta", "dA_log", "dB", "dC", "dD", "dz", "dh0")


@pytest.fixture(autouse=True)
def _announce(request):
    announce(request.node.nodeid)
    yield


def _case(w):
    inp = gen.generate(w)
    u = oracle.conv1d_silu(inp["x"], inp["w_conv"], inp["b_conv"], batch=w.batch,
                           seq_len=w.seq_len).astype(np.float32)
    dout = gen.cotangent(w)
    d = {k: dev(v) for k, v in inp.items()}
    args = (dev(u), d["delta"], d["A_log"], d["B"], d["C"], d["D_vec"], d["z"], d.get("h0"),
            dev(dout))
    return args


@pytest.mark.parametrize("disc", ("zoh", "euler"))
def test_noalloc_backward_matches_workspace_entry_point(disc):
    import torch
    big = gen.SMALL.with_(name="noalloc_big", batch=2, seq_len=1500, d_inner=300, h0=True)
    small = gen.SMALL.with_(name="noalloc_small", batch=1, seq_len=333, d_inner=70, h0=True,
                            seed_index=7)
    for w in (big, small):
        need = mss.workspace_bytes(mss.OP_SELECTIVE_SCAN_BACKWARD, batch=w.batch,
                                   seq_len=w.seq_len, d_inner=w.d_inner, d_state=w.d_state)
        assert 0 < need <= mss.NOALLOC_SCRATCH_BYTES
    cb, cs = _case(big), _case(small)
    kw = lambda w: dict(batch=w.batch, seq_len=w.seq_len, disc=disc, need_dh0=True)
    # two calls in a row on the static array, the second smaller
    g_big = mss.selective_scan_backward_noalloc(*cb, **kw(big))
    g_small = mss.selective_scan_backward_noalloc(*cs, **kw(small))
    torch.cuda.synchronize()
    r_big = mss.selective_scan_backward(*cb, **kw(big))
    r_small = mss.selective_scan_backward(*cs, **kw(small))
    torch.cuda.synchronize()
    for name, g, r in (("first", g_big, r_big), ("second, smaller", g_small, r_small)):
        for k in KEYS:
            got, want = host(g[k]), host(r[k])
            assert np.array_equal(got, want), f"{name}: {k} differs"
            assert_close(got, want, f"{name}: {k}")
    # larger again after the workspace entry point ran: same answer as before
    g_again = mss.selective_scan_backward_noalloc(*cb, **kw(big))
    torch.cuda.synchronize()
    for k in KEYS:
        assert np.array_equal(host(g_again[k]), host(r_big[k])), k


@pytest.mark.parametrize("disc", ("zoh", "euler"))
def test_noalloc_backward_exact_matches_workspace_entry_point(disc):
    """MSS_FLAG_EXACT (one segment per channel tile, a workspace laid out for
    it) on the static array, right after a split call has left its own
    contents there: bit for bit the workspace entry point's answer."""
    import torch
    w = gen.SMALL.with_(name="noalloc_exact", batch=2, seq_len=900, d_inner=100, h0=True,
                        seed_index=9)
    c = _case(w)
    kw = dict(batch=w.batch, seq_len=w.seq_len, disc=disc, need_dh0=True)
    mss.selective_scan_backward_noalloc(*c, **kw)
    g = mss.selective_scan_backward_noalloc(*c, exact=True, **kw)
    r = mss.selective_scan_backward(*c, exact=True, **kw)
    torch.cuda.synchronize()
    for k in KEYS:
        assert np.array_equal(host(g[k]), host(r[k])), k


def test_noalloc_backward_refuses_past_the_array():
    import torch
    w = gen.MAMBA_130M
    need = mss.workspace_bytes(mss.OP_SELECTIVE_SCAN_BACKWARD, batch=w.batch, seq_len=w.seq_len,
                               d_inner=w.d_inner, d_state=w.d_state)
    assert need > mss.NOALLOC_SCRATCH_BYTES
    # with the forward's checkpoints the same problem fits
    assert mss.workspace_bytes(mss.OP_SELECTIVE_SCAN_BACKWARD, batch=w.batch, seq_len=w.seq_len,
                               d_inner=w.d_inner, d_state=w.d_state,
                               ckpt8=True) < mss.NOALLOC_SCRATCH_BYTES
    M, D, N = w.M, w.d_inner, w.d_state
    z = torch.zeros
    args = (z((M, D), device="cuda"), z((M, D), device="cuda"), z((D, N), device="cuda"),
            z((M, N), device="cuda"), z((M, N), device="cuda"), None, None, None,
            z((M, D), device="cuda"))
    with pytest.raises(mss.MssError) as e:
        mss.selective_scan_backward_noalloc(*args, batch=w.batch, seq_len=w.seq_len,
                                            disc="zoh")
    assert e.value.status == mss.MSS_ESCRATCH
