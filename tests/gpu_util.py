"""Helpers shared by the GPU tests: device transfer and the tolerance metric."""
from __future__ import annotations

import sys

import numpy as np

TOL = 1e-4  # max relative error, fp32 GPU vs fp64 oracle


# pytest's capture manager, set by conftest.pytest_configure: announce
# suspends capture through it so the line reaches the real stderr at once.
_capture = None


def announce(msg: str):
    """Print a progress line to the terminal's stderr, flushed, with pytest's
    output capture suspended, so it shows even when the test passes or the
    process dies in the next GPU call."""
    if _capture is not None:
        with _capture.global_and_fixture_disabled():
            sys.stderr.write(f"[gpu] {msg}\n")
            sys.stderr.flush()
    else:
        sys.stderr.write(f"[gpu] {msg}\n")
        sys.stderr.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nan_like(shape):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def host(t):
    return t.detach().cpu().numpy().astype(np.float64)


def rel_err(got, want) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o)): relative error above the tensor's
    rms, absolute error scaled by the rms below it (where the output cancels).
    Non-finite GPU values where the oracle is finite count as infinite error."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if want.size == 0:
        return 0.0
    fin = np.isfinite(want)
    if not np.isfinite(got[fin]).all():
        return float("inf")
    w = want[fin]
    rms = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
    den = np.maximum(np.abs(w), rms)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(got[fin] - w) / den).max())


def assert_close(got, want, what, tol=TOL):
    e = rel_err(got, want)
    assert e <= tol, f"{what}: max relative error {e:.3e} > {tol:.1e}"
    return e
