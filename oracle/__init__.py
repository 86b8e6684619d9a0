"""CPU oracle for the Mamba-1 (S6) block core -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does, and shares no code with it.

Thin ctypes wrapper over ``oracle.c`` (plain fp64 C loops).  Every function
takes the fp32 numpy inputs the GPU receives and returns fp64 numpy outputs.
See ``oracle.c`` for the formulas and the passages of the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ZOH = 0
EULER = 1
DISC = {"zoh": ZOH, "euler": EULER}

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
          "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with gcc (no HIP involved)."""
    cmd = ["gcc", *CFLAGS, *extra, "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if needed) and return the ctypes library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(lib):
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_conv1d_silu.argtypes = [i64, i64, i64, i64, p, p, p, p, i32]
    lib.oracle_selective_scan.argtypes = [i64, i64, i64, i64, i32, p, p, p, p, p, p, p, p,
                                          p, i64, p, p, p, i32]
    lib.oracle_mamba1_core.argtypes = [i64, i64, i64, i64, i64, i32, p, p, p, p, p, p, p, p,
                                       p, p, p, i64, p, p, p, i32]
    lib.oracle_selective_step.argtypes = [i64, i64, i64, i64, i32, p, p, p, p, p, p, p, p, p,
                                          p, p, p, i64, p, p, p, i32]
    lib.oracle_selective_scan_backward.argtypes = [i64, i64, i64, i64, i32] + [p] * 17 + [i32]
    lib.oracle_conv1d_silu_backward.argtypes = [i64, i64, i64, i64] + [p] * 7 + [i32]
    lib.oracle_ssd_scan.argtypes = [i64] * 6 + [i32] + [p] * 10 + [i32]
    for f in (lib.oracle_conv1d_silu, lib.oracle_selective_scan, lib.oracle_mamba1_core,
              lib.oracle_selective_step, lib.oracle_selective_scan_backward,
              lib.oracle_conv1d_silu_backward, lib.oracle_ssd_scan):
        f.restype = ctypes.c_int
    return lib


def _f32(a, name, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {a.shape}")
    return a


def _f64(a, name, shape=None):
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _disc(disc) -> int:
    if isinstance(disc, str):
        return DISC[disc.lower()]
    if disc not in (ZOH, EULER):
        raise ValueError("disc must be 'zoh' or 'euler'")
    return int(disc)


def _cols(cols):
    if cols is None:
        return None, 0
    c = np.ascontiguousarray(cols, dtype=np.int64)
    return c, int(c.size)


def conv1d_silu(x, w_conv, b_conv=None, *, batch, seq_len, nthreads=0, lib=None):
    """u = SiLU(causal depthwise conv1d(x)) in fp64, layout (batch*seq_len, D)."""
    D = x.shape[-1]
    K = w_conv.shape[1]
    x = _f32(x, "x", (batch * seq_len, D))
    w = _f32(w_conv, "w_conv", (D, K))
    b = _f32(b_conv, "b_conv", (D,))
    u = np.empty((batch * seq_len, D), dtype=np.float64)
    rc = (lib or load()).oracle_conv1d_silu(batch, seq_len, D, K, _ptr(x), _ptr(w), _ptr(b), _ptr(u),
                                   nthreads)
    if rc != 0:
        raise ValueError(f"oracle_conv1d_silu failed ({rc})")
    return u


def _scan_outputs(B, L, D, N, cols, h_cache, h_last):
    if cols is None:
        y = np.empty((B * L, D), dtype=np.float64)
        hc = np.empty((B, L, D, N), dtype=np.float64) if h_cache else None
        hl = np.empty((B, D, N), dtype=np.float64) if h_last else None
    else:
        nc = cols.size
        y = np.empty((nc, L), dtype=np.float64)
        hc = np.empty((nc, L, N), dtype=np.float64) if h_cache else None
        hl = np.empty((nc, N), dtype=np.float64) if h_last else None
    return y, hc, hl


def selective_scan(u, delta, A_log, B, C, D_vec=None, z=None, h0=None, *, batch, seq_len,
                   disc, cols=None, h_cache=False, h_last=False, nthreads=0, lib=None):
    """Selective scan + gate on a given u.  Returns (y, h_cache, h_last).

    ``cols``: optional list of column ids b*D + d; then outputs are compact
    (ncols, L) / (ncols, L, N) / (ncols, N).
    """
    Dn, N = A_log.shape
    M = batch * seq_len
    args = [_f32(u, "u", (M, Dn)), _f32(delta, "delta", (M, Dn)), _f32(A_log, "A_log", (Dn, N)),
            _f32(B, "B", (M, N)), _f32(C, "C", (M, N)), _f32(D_vec, "D_vec", (Dn,)),
            _f32(z, "z", (M, Dn)), _f32(h0, "h0", (batch, Dn, N))]
    cols, nc = _cols(cols)
    y, hc, hl = _scan_outputs(batch, seq_len, Dn, N, cols, h_cache, h_last)
    rc = (lib or load()).oracle_selective_scan(batch, seq_len, Dn, N, _disc(disc), *map(_ptr, args),
                                      _ptr(cols), nc, _ptr(y), _ptr(hc), _ptr(hl), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_selective_scan failed ({rc})")
    return y, hc, hl


def mamba1_core(x, w_conv, b_conv, delta, A_log, B, C, D_vec=None, z=None, h0=None, *,
                batch, seq_len, disc, cols=None, h_cache=False, h_last=False, nthreads=0,
                lib=None):
    """Conv1d + SiLU + selective scan + gate from x.  Returns (y, h_cache, h_last)."""
    Dn, N = A_log.shape
    K = w_conv.shape[1]
    M = batch * seq_len
    args = [_f32(x, "x", (M, Dn)), _f32(w_conv, "w_conv", (Dn, K)),
            _f32(b_conv, "b_conv", (Dn,)), _f32(delta, "delta", (M, Dn)),
            _f32(A_log, "A_log", (Dn, N)), _f32(B, "B", (M, N)), _f32(C, "C", (M, N)),
            _f32(D_vec, "D_vec", (Dn,)), _f32(z, "z", (M, Dn)), _f32(h0, "h0", (batch, Dn, N))]
    cols, nc = _cols(cols)
    y, hc, hl = _scan_outputs(batch, seq_len, Dn, N, cols, h_cache, h_last)
    rc = (lib or load()).oracle_mamba1_core(batch, seq_len, Dn, N, K, _disc(disc), *map(_ptr, args),
                                   _ptr(cols), nc, _ptr(y), _ptr(hc), _ptr(hl), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_mamba1_core failed ({rc})")
    return y, hc, hl


def selective_step(x, z, delta, A_log, B, C, D_vec, w_conv, b_conv, conv_state, h, *, disc,
                   cols=None, nthreads=0, lib=None):
    """One recurrent step.  Returns (y, conv_state_new, h_new) in fp64.

    Full layout: x, z, delta (Bt, D); B, C (Bt, N); conv_state (Bt, K-1, D);
    h (Bt, D, N).  With ``cols`` the state and outputs are compact:
    conv_state (ncols, K-1), h (ncols, N), y (ncols,).
    """
    Bt, Dn = x.shape
    N = A_log.shape[1]
    K = w_conv.shape[1]
    cols, nc = _cols(cols)
    if cols is None:
        cs_shape, h_shape, y_shape = (Bt, K - 1, Dn), (Bt, Dn, N), (Bt, Dn)
    else:
        cs_shape, h_shape, y_shape = (nc, K - 1), (nc, N), (nc,)
    args = [_f32(x, "x", (Bt, Dn)), _f32(z, "z", (Bt, Dn)), _f32(delta, "delta", (Bt, Dn)),
            _f32(A_log, "A_log", (Dn, N)), _f32(B, "B", (Bt, N)), _f32(C, "C", (Bt, N)),
            _f32(D_vec, "D_vec", (Dn,)), _f32(w_conv, "w_conv", (Dn, K)),
            _f32(b_conv, "b_conv", (Dn,)), _f64(conv_state, "conv_state", cs_shape),
            _f64(h, "h", h_shape)]
    y = np.empty(y_shape, dtype=np.float64)
    cs_out = np.empty(cs_shape, dtype=np.float64)
    h_out = np.empty(h_shape, dtype=np.float64)
    rc = (lib or load()).oracle_selective_step(Bt, Dn, N, K, _disc(disc), *map(_ptr, args), _ptr(cols),
                                      nc, _ptr(y), _ptr(cs_out), _ptr(h_out), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_selective_step failed ({rc})")
    return y, cs_out, h_out


def selective_scan_backward(u, delta, A_log, B, C, D_vec, z, h0, dout, *, batch, seq_len, disc,
                            nthreads=0, lib=None):
    """Gradients of the gated scan output against ``dout`` (fp64 dict).

    Keys: du, ddelta, dz (or None when z is None) (M, D); dA_log (D, N);
    dB, dC (M, N); dD (D,); dh0 (batch, D, N).  ``du`` is the gradient that
    reaches u through the scan only.
    """
    Dn, N = A_log.shape
    M = batch * seq_len
    args = [_f32(u, "u", (M, Dn)), _f32(delta, "delta", (M, Dn)), _f32(A_log, "A_log", (Dn, N)),
            _f32(B, "B", (M, N)), _f32(C, "C", (M, N)), _f32(D_vec, "D_vec", (Dn,)),
            _f32(z, "z", (M, Dn)), _f32(h0, "h0", (batch, Dn, N)),
            _f32(dout, "dout", (M, Dn))]
    out = {"du": np.empty((M, Dn)), "ddelta": np.empty((M, Dn)), "dA_log": np.empty((Dn, N)),
           "dB": np.empty((M, N)), "dC": np.empty((M, N)), "dD": np.empty((Dn,)),
           "dz": np.empty((M, Dn)) if z is not None else None,
           "dh0": np.empty((batch, Dn, N))}
    rc = (lib or load()).oracle_selective_scan_backward(
        batch, seq_len, Dn, N, _disc(disc), *map(_ptr, args),
        *(_ptr(out[k]) for k in ("du", "ddelta", "dA_log", "dB", "dC", "dD", "dz", "dh0")),
        nthreads)
    if rc != 0:
        raise ValueError(f"oracle_selective_scan_backward failed ({rc})")
    return out


def conv1d_silu_backward(x, w_conv, b_conv, du, *, batch, seq_len, nthreads=0, lib=None):
    """Gradients of u = SiLU(conv1d(x)) against ``du``: (dx, dw_conv, db_conv), fp64."""
    D = x.shape[-1]
    K = w_conv.shape[1]
    M = batch * seq_len
    args = [_f32(x, "x", (M, D)), _f32(w_conv, "w_conv", (D, K)), _f32(b_conv, "b_conv", (D,)),
            _f32(du, "du", (M, D))]
    dx, dw, db = np.empty((M, D)), np.empty((D, K)), np.empty((D,))
    rc = (lib or load()).oracle_conv1d_silu_backward(batch, seq_len, D, K, *map(_ptr, args),
                                                     _ptr(dx), _ptr(dw), _ptr(db), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_conv1d_silu_backward failed ({rc})")
    return dx, dw, db


def ssd_scan(x, dt, A_log, B, C, D_vec=None, dt_bias=None, h0=None, *, batch, seq_len,
             n_heads, head_dim, d_state, n_groups=1, disc, h_last=False, nthreads=0, lib=None):
    """Mamba-2 SSD scan in fp64.  Returns (y (M, H*P), h_last (batch, H, P, N) or None)."""
    H, P, N, G = n_heads, head_dim, d_state, n_groups
    M = batch * seq_len
    args = [_f32(x, "x", (M, H * P)), _f32(dt, "dt", (M, H)), _f32(A_log, "A_log", (H,)),
            _f32(B, "B", (M, G * N)), _f32(C, "C", (M, G * N)), _f32(D_vec, "D_vec", (H,)),
            _f32(dt_bias, "dt_bias", (H,)), _f32(h0, "h0", (batch, H, P, N))]
    y = np.empty((M, H * P))
    hl = np.empty((batch, H, P, N)) if h_last else None
    rc = (lib or load()).oracle_ssd_scan(batch, seq_len, H, P, N, G, _disc(disc), *map(_ptr, args), _ptr(y),
                                         _ptr(hl), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_ssd_scan failed ({rc})")
    return y, hl


class Bound:
    """The same API bound to one specific oracle build (used by the tests that
    check the pins against deliberately broken copies of ``oracle.c``)."""

    def __init__(self, lib):
        self.lib = lib

    def conv1d_silu(self, *a, **k):
        return conv1d_silu(*a, lib=self.lib, **k)

    def selective_scan(self, *a, **k):
        return selective_scan(*a, lib=self.lib, **k)

    def mamba1_core(self, *a, **k):
        return mamba1_core(*a, lib=self.lib, **k)

    def selective_step(self, *a, **k):
        return selective_step(*a, lib=self.lib, **k)

    def selective_scan_backward(self, *a, **k):
        return selective_scan_backward(*a, lib=self.lib, **k)

    def conv1d_silu_backward(self, *a, **k):
        return conv1d_silu_backward(*a, lib=self.lib, **k)

    def ssd_scan(self, *a, **k):
        return ssd_scan(*a, lib=self.lib, **k)


def default() -> Bound:
    return Bound(load())
