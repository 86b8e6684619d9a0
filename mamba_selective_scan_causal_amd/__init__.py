"""MI355X-native Mamba-1 (S6) block core: Python binding of libmss.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmss.so`` (built in-tree by ``build.py``); PyTorch supplies
device memory and the current stream.  There is no fallback: if the library
is missing or a call fails, an exception is raised.

Layouts (fp32, contiguous, on the current CUDA/HIP device):
  x, z, delta, u, y : (batch*seq_len, D)     B, C : (batch*seq_len, N)
  A_log : (D, N)   D_vec, b_conv : (D,)   w_conv : (D, K)
  h0, h_last : (batch, D, N)   h_cache : (batch, seq_len, D, N)
Single-token step: x, z, delta, y : (batch, D); B, C : (batch, N);
  conv_state : (batch, K-1, D) oldest first; h : (batch, D, N).
"""
from __future__ import annotations

import ctypes
import os

from . import inputs  # noqa: F401  (seeded synthetic inputs; no method arithmetic)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmss.so")

ZOH = 0
EULER = 1
_DISC = {"zoh": ZOH, "euler": EULER, ZOH: ZOH, EULER: EULER}

MSS_OK = 0


class MssError(RuntimeError):
    def __init__(self, fn, status, msg, hip_error=0):
        super().__init__(f"{fn} failed: status {status} ({msg})"
                         + (f", hipError {hip_error}" if hip_error else ""))
        self.status = status
        self.hip_error = hip_error


class Dims(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("d_conv", ctypes.c_int64)]


FLAG_EXACT = 1          # no time split: the plain sequential recurrence
FLAG_CKPT8 = 2          # state checkpoints every 8 steps (forward h_cache / backward h_ckpt)


def make_dims(batch, seq_len, d_inner, d_state, d_conv=1, exact=False, ckpt8=False) -> Dims:
    flags = (FLAG_EXACT if exact else 0) | (FLAG_CKPT8 if ckpt8 else 0)
    return Dims(ctypes.sizeof(Dims), flags, batch, seq_len, d_inner, d_state, d_conv)


class Strides(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("x", ctypes.c_int64), ("z", ctypes.c_int64), ("delta", ctypes.c_int64),
                ("B", ctypes.c_int64), ("C", ctypes.c_int64), ("y", ctypes.c_int64)]


def make_strides(x, z, delta, B, C, y) -> Strides:
    return Strides(ctypes.sizeof(Strides), 0, x, z, delta, B, C, y)


class SsdDims(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("n_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("d_state", ctypes.c_int64), ("n_groups", ctypes.c_int64)]


def make_ssd_dims(batch, seq_len, n_heads, head_dim, d_state, n_groups=1, exact=False) -> SsdDims:
    return SsdDims(ctypes.sizeof(SsdDims), FLAG_EXACT if exact else 0, batch, seq_len, n_heads,
                   head_dim, d_state, n_groups)


EXPORTS = ("mss_conv1d_silu", "mss_selective_scan", "mss_mamba1_core", "mss_selective_step",
           "mss_selective_scan_strided", "mss_mamba1_core_strided",
           "mss_workspace_bytes", "mss_selective_scan_backward", "mss_conv1d_silu_backward",
           "mss_ssd_scan", "mss_time_split", "mss_ssd_time_split",
           "mss_selective_scan_backward_noalloc",
           "mss_strerror", "mss_version", "mss_last_hip_error")

OP_SELECTIVE_SCAN_BACKWARD = 1
OP_CONV1D_SILU_BACKWARD = 2
OP_SELECTIVE_SCAN = 3
NOALLOC_SCRATCH_BYTES = 256 << 20     # MSS_NOALLOC_SCRATCH_BYTES
MSS_ESCRATCH = -6

_lib = None


def lib():
    """The loaded libmss (ctypes).  Raises if the HIP library is not built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime (soname libamdhip64.so.7, file name
        # libamdhip64.so).  Loaded first, it also serves libmss's dependency;
        # loading libmss first would bring in a second runtime from the ROCm
        # install, which does not see torch's device memory.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mamba_selective_scan_causal_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i = ctypes.c_void_p, ctypes.c_int
        dp = ctypes.POINTER(Dims)
        L.mss_conv1d_silu.argtypes = [dp, p, p, p, p, p]
        L.mss_selective_scan.argtypes = [dp, i, p, p, p, p, p, p, p, p, p, p, p, p]
        L.mss_mamba1_core.argtypes = [dp, i, p, p, p, p, p, p, p, p, p, p, p, p, p, p]
        L.mss_selective_step.argtypes = [dp, i, p, p, p, p, p, p, p, p, p, p, p, p, p]
        sp = ctypes.POINTER(Strides)
        L.mss_selective_scan_strided.argtypes = [dp, sp, i] + [p] * 12
        L.mss_mamba1_core_strided.argtypes = [dp, sp, i] + [p] * 14
        sz = ctypes.c_size_t
        L.mss_workspace_bytes.argtypes = [dp, i, ctypes.POINTER(sz)]
        L.mss_selective_scan_backward.argtypes = [dp, i] + [p] * 19 + [sz, p]
        L.mss_selective_scan_backward_noalloc.argtypes = [dp, i] + [p] * 18
        L.mss_conv1d_silu_backward.argtypes = [dp] + [p] * 8 + [sz, p]
        L.mss_ssd_scan.argtypes = [ctypes.POINTER(SsdDims), i] + [p] * 11
        L.mss_time_split.argtypes = [dp, i, ctypes.POINTER(ctypes.c_int64)]
        L.mss_ssd_time_split.argtypes = [ctypes.POINTER(SsdDims), ctypes.POINTER(ctypes.c_int64)]
        for f in ("mss_conv1d_silu", "mss_selective_scan", "mss_mamba1_core",
                  "mss_selective_step", "mss_selective_scan_strided", "mss_mamba1_core_strided",
                  "mss_workspace_bytes", "mss_selective_scan_backward",
                  "mss_conv1d_silu_backward", "mss_ssd_scan", "mss_time_split",
                  "mss_ssd_time_split", "mss_selective_scan_backward_noalloc", "mss_version",
                  "mss_last_hip_error"):
            getattr(L, f).restype = ctypes.c_int
        L.mss_strerror.argtypes = [ctypes.c_int]
        L.mss_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn, status):
    if status != MSS_OK:
        L = lib()
        raise MssError(fn, status, L.mss_strerror(status).decode(), L.mss_last_hip_error())


def _disc(disc) -> int:
    key = disc.lower() if isinstance(disc, str) else disc
    if key not in _DISC:
        raise ValueError("disc must be 'zoh' or 'euler'")
    return _DISC[key]


def _torch():
    import torch
    return torch


def _ptr(t, name, shape, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    _same_device(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr() or None


def _rows(t, name, rows, cols, required=True):
    """(pointer, row stride) of a (rows, cols) fp32 GPU tensor whose rows may be
    strided (a column slice of a wider buffer); columns must be unit-stride."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None, cols
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda:
        raise TypeError(f"{name} must be a float32 GPU tensor")
    _same_device(t, name)
    if tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name}: expected shape {(rows, cols)}, got {tuple(t.shape)}")
    if rows > 0 and cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: columns must be contiguous")
    ld = t.stride(0) if rows > 1 else cols
    return (t.data_ptr() or None), ld


def _same_device(t, name):
    # the kernels run on the current device: every tensor must live there
    dev = _torch().cuda.current_device()
    if t.device.index != dev:
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{dev}")


def _dense(*ts):
    return all(t is None or t.is_contiguous() for t in ts)


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    if s.device.index != torch.cuda.current_device():
        raise ValueError(f"stream is on {s.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, like):
    return _torch().empty(shape, dtype=like.dtype, device=like.device)


def conv1d_silu(x, w_conv, b_conv=None, *, batch, seq_len, out=None, stream=None):
    """u = SiLU(causal depthwise conv1d(x) + b_conv), (batch*seq_len, D)."""
    D, K = w_conv.shape
    M = batch * seq_len
    u = out if out is not None else _empty((M, D), x)
    dims = make_dims(batch, seq_len, D, 1, K)
    _check("mss_conv1d_silu", lib().mss_conv1d_silu(
        ctypes.byref(dims), _ptr(x, "x", (M, D)), _ptr(w_conv, "w_conv", (D, K)),
        _ptr(b_conv, "b_conv", (D,), False), _ptr(u, "u", (M, D)), _stream(stream)))
    return u


def ckpt_steps(seq_len) -> int:
    """Rows of an 8-step checkpoint tensor: ceil(seq_len / 8)."""
    return (seq_len + 7) // 8


def _scan_outputs(x, batch, seq_len, D, N, out, h_cache, h_last, ckpt8=False):
    M = batch * seq_len
    y = out if out is not None else _empty((M, D), x)
    Lc = ckpt_steps(seq_len) if ckpt8 else seq_len
    hc = (h_cache if not isinstance(h_cache, bool) else
          (_empty((batch, Lc, D, N), x) if h_cache else None))
    hl = (h_last if not isinstance(h_last, bool) else
          (_empty((batch, D, N), x) if h_last else None))
    return y, hc, hl


def selective_scan(u, delta, A_log, B, C, D_vec=None, z=None, h0=None, *, batch, seq_len, disc,
                   h_cache=False, h_last=False, out=None, stream=None, exact=False, ckpt8=False):
    """Selective scan + gate on a given u.  Returns (y, h_cache, h_last).

    ``h_cache`` / ``h_last``: False (skip), True (allocate) or an output tensor.
    u, delta, z, B, C and ``out`` may be row-strided views (column slices).
    ``exact``: no time split (the plain sequential recurrence, less parallel).
    ``ckpt8``: h_cache is (batch, ceil(seq_len/8), D, N), the state entering
    steps 0, 8, 16, ... (the backward's checkpoints)."""
    D, N = A_log.shape
    M = batch * seq_len
    Lc = ckpt_steps(seq_len) if ckpt8 else seq_len
    y, hc, hl = _scan_outputs(u, batch, seq_len, D, N, out, h_cache, h_last, ckpt8)
    dims = make_dims(batch, seq_len, D, N, 1, exact, ckpt8)
    common = (_ptr(A_log, "A_log", (D, N)),)
    tail = (_ptr(D_vec, "D_vec", (D,), False),)
    if _dense(u, delta, B, C, z, y):
        _check("mss_selective_scan", lib().mss_selective_scan(
            ctypes.byref(dims), _disc(disc), _ptr(u, "u", (M, D)), _ptr(delta, "delta", (M, D)),
            *common, _ptr(B, "B", (M, N)), _ptr(C, "C", (M, N)), *tail,
            _ptr(z, "z", (M, D), False), _ptr(h0, "h0", (batch, D, N), False),
            _ptr(y, "y", (M, D)), _ptr(hc, "h_cache", (batch, Lc, D, N), False),
            _ptr(hl, "h_last", (batch, D, N), False), _stream(stream)))
        return y, hc, hl
    pu, lu = _rows(u, "u", M, D)
    pd, ldd = _rows(delta, "delta", M, D)
    pb, lb = _rows(B, "B", M, N)
    pc, lc = _rows(C, "C", M, N)
    pz, lz = _rows(z, "z", M, D, False)
    py, ly = _rows(y, "y", M, D)
    st = make_strides(lu, lz, ldd, lb, lc, ly)
    _check("mss_selective_scan_strided", lib().mss_selective_scan_strided(
        ctypes.byref(dims), ctypes.byref(st), _disc(disc), pu, pd, *common, pb, pc, *tail, pz,
        _ptr(h0, "h0", (batch, D, N), False), py,
        _ptr(hc, "h_cache", (batch, Lc, D, N), False),
        _ptr(hl, "h_last", (batch, D, N), False), _stream(stream)))
    return y, hc, hl


def mamba1_core(x, w_conv, b_conv, delta, A_log, B, C, D_vec=None, z=None, h0=None, *, batch,
                seq_len, disc, h_cache=False, h_last=False, out=None, stream=None, exact=False,
                ckpt8=False):
    """Fused conv1d + SiLU + selective scan + gate from x.  Returns (y, h_cache, h_last).

    x, delta, z, B, C and ``out`` may be row-strided views (column slices).
    ``exact``: no time split (the plain sequential recurrence, less parallel).
    ``ckpt8``: h_cache is the state entering every 8th step (see selective_scan)."""
    D, N = A_log.shape
    K = w_conv.shape[1]
    M = batch * seq_len
    Lc = ckpt_steps(seq_len) if ckpt8 else seq_len
    y, hc, hl = _scan_outputs(x, batch, seq_len, D, N, out, h_cache, h_last, ckpt8)
    dims = make_dims(batch, seq_len, D, N, K, exact, ckpt8)
    conv = (_ptr(w_conv, "w_conv", (D, K)), _ptr(b_conv, "b_conv", (D,), False))
    if _dense(x, delta, B, C, z, y):
        _check("mss_mamba1_core", lib().mss_mamba1_core(
            ctypes.byref(dims), _disc(disc), _ptr(x, "x", (M, D)), *conv,
            _ptr(delta, "delta", (M, D)), _ptr(A_log, "A_log", (D, N)), _ptr(B, "B", (M, N)),
            _ptr(C, "C", (M, N)), _ptr(D_vec, "D_vec", (D,), False), _ptr(z, "z", (M, D), False),
            _ptr(h0, "h0", (batch, D, N), False), _ptr(y, "y", (M, D)),
            _ptr(hc, "h_cache", (batch, Lc, D, N), False),
            _ptr(hl, "h_last", (batch, D, N), False), _stream(stream)))
        return y, hc, hl
    px, lx = _rows(x, "x", M, D)
    pd, ldd = _rows(delta, "delta", M, D)
    pb, lb = _rows(B, "B", M, N)
    pc, lc = _rows(C, "C", M, N)
    pz, lz = _rows(z, "z", M, D, False)
    py, ly = _rows(y, "y", M, D)
    st = make_strides(lx, lz, ldd, lb, lc, ly)
    _check("mss_mamba1_core_strided", lib().mss_mamba1_core_strided(
        ctypes.byref(dims), ctypes.byref(st), _disc(disc), px, *conv, pd,
        _ptr(A_log, "A_log", (D, N)), pb, pc, _ptr(D_vec, "D_vec", (D,), False), pz,
        _ptr(h0, "h0", (batch, D, N), False), py,
        _ptr(hc, "h_cache", (batch, Lc, D, N), False),
        _ptr(hl, "h_last", (batch, D, N), False), _stream(stream)))
    return y, hc, hl


def selective_step(x, z, delta, A_log, B, C, D_vec, w_conv, b_conv, conv_state, h, *, disc,
                   out=None, stream=None):
    """One decode step; updates ``conv_state`` and ``h`` in place.  Returns y (batch, D)."""
    batch, D = x.shape
    N = A_log.shape[1]
    K = w_conv.shape[1]
    y = out if out is not None else _empty((batch, D), x)
    dims = make_dims(batch, 1, D, N, K)
    _check("mss_selective_step", lib().mss_selective_step(
        ctypes.byref(dims), _disc(disc), _ptr(x, "x", (batch, D)),
        _ptr(z, "z", (batch, D), False), _ptr(delta, "delta", (batch, D)),
        _ptr(A_log, "A_log", (D, N)), _ptr(B, "B", (batch, N)), _ptr(C, "C", (batch, N)),
        _ptr(D_vec, "D_vec", (D,), False), _ptr(w_conv, "w_conv", (D, K)),
        _ptr(b_conv, "b_conv", (D,), False),
        _ptr(conv_state, "conv_state", (batch, K - 1, D), K > 1),
        _ptr(h, "h", (batch, D, N)), _ptr(y, "y", (batch, D)), _stream(stream)))
    return y


def workspace_bytes(op, *, batch, seq_len, d_inner, d_state, d_conv=1, exact=False,
                    ckpt8=False) -> int:
    """Workspace bytes a backward entry point needs (``op``: OP_* constant;
    ``ckpt8``: the scan backward is given the forward's checkpoints)."""
    dims = make_dims(batch, seq_len, d_inner, d_state, d_conv, exact, ckpt8)
    n = ctypes.c_size_t(0)
    _check("mss_workspace_bytes", lib().mss_workspace_bytes(ctypes.byref(dims), op,
                                                             ctypes.byref(n)))
    return int(n.value)


def _workspace(op, like, workspace, stream, **dims):
    """The caller's workspace (a uint8 GPU tensor), or a fresh one of the size
    the library asks for; returns (pointer, bytes, tensor)."""
    need = workspace_bytes(op, **dims)
    if workspace is None:
        if need == 0:
            return None, 0, None
        # 256 bytes of slack so that the pointer can be aligned to 256.
        workspace = _torch().empty(need + 256, dtype=_torch().uint8, device=like.device)
        if stream is not None:
            # freed when the caller drops the result: keep it alive for the
            # work queued on that stream
            workspace.record_stream(stream)
    if workspace.dtype != _torch().uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 GPU tensor")
    _same_device(workspace, "workspace")
    base = workspace.data_ptr()
    pad = (-base) % 256
    return base + pad, max(0, workspace.numel() - pad), workspace


def time_split(op, *, batch, seq_len, d_inner, d_state, d_conv=1, exact=False) -> int:
    """Segment length in steps of the flattened (channel tile, t) space that
    ``op`` (OP_SELECTIVE_SCAN or OP_SELECTIVE_SCAN_BACKWARD) uses."""
    dims = make_dims(batch, seq_len, d_inner, d_state, d_conv, exact)
    n = ctypes.c_int64(0)
    _check("mss_time_split", lib().mss_time_split(ctypes.byref(dims), op, ctypes.byref(n)))
    return int(n.value)


def ssd_time_split(*, batch, seq_len, n_heads, head_dim, d_state, n_groups=1,
                   exact=False) -> int:
    """Segment length in steps of every (batch row, head) sequence of ssd_scan."""
    dims = make_ssd_dims(batch, seq_len, n_heads, head_dim, d_state, n_groups, exact)
    n = ctypes.c_int64(0)
    _check("mss_ssd_time_split", lib().mss_ssd_time_split(ctypes.byref(dims), ctypes.byref(n)))
    return int(n.value)


def selective_scan_backward(u, delta, A_log, B, C, D_vec, z, h0, dout, *, batch, seq_len, disc,
                            need_dh0=False, workspace=None, stream=None, exact=False,
                            h_ckpt=None):
    """Gradients of ``selective_scan``'s output against ``dout`` (batch*seq_len, D).

    Returns a dict: du, ddelta (M, D); dA_log (D, N); dB, dC (M, N);
    dD (D,) or None when D_vec is None; dz (M, D) or None when z is None;
    dh0 (batch, D, N) when ``need_dh0``.  ``workspace``: optional uint8 GPU
    tensor of at least ``workspace_bytes(OP_SELECTIVE_SCAN_BACKWARD, ...)``
    + 256 bytes (allocated here when omitted).  ``exact``: no time split.
    ``h_ckpt``: the forward's 8-step checkpoints (``h_cache`` of a forward
    call with ``ckpt8=True``), from which every 8-step block starts.
    """
    D, N = A_log.shape
    M = batch * seq_len
    g = {"du": _empty((M, D), u), "ddelta": _empty((M, D), u), "dA_log": _empty((D, N), u),
         "dB": _empty((M, N), u), "dC": _empty((M, N), u),
         "dD": _empty((D,), u) if D_vec is not None else None,
         "dz": _empty((M, D), u) if z is not None else None,
         "dh0": _empty((batch, D, N), u) if need_dh0 else None}
    ck = h_ckpt is not None
    wp, wn, _keep = _workspace(OP_SELECTIVE_SCAN_BACKWARD, u, workspace, stream, batch=batch,
                               seq_len=seq_len, d_inner=D, d_state=N, exact=exact, ckpt8=ck)
    dims = make_dims(batch, seq_len, D, N, 1, exact, ck)
    _check("mss_selective_scan_backward", lib().mss_selective_scan_backward(
        ctypes.byref(dims), _disc(disc), _ptr(u, "u", (M, D)), _ptr(delta, "delta", (M, D)),
        _ptr(A_log, "A_log", (D, N)), _ptr(B, "B", (M, N)), _ptr(C, "C", (M, N)),
        _ptr(D_vec, "D_vec", (D,), False), _ptr(z, "z", (M, D), False),
        _ptr(h0, "h0", (batch, D, N), False),
        _ptr(h_ckpt, "h_ckpt", (batch, ckpt_steps(seq_len), D, N), False),
        _ptr(dout, "dout", (M, D)),
        _ptr(g["du"], "du", (M, D)), _ptr(g["ddelta"], "ddelta", (M, D)),
        _ptr(g["dA_log"], "dA_log", (D, N)), _ptr(g["dB"], "dB", (M, N)),
        _ptr(g["dC"], "dC", (M, N)), _ptr(g["dD"], "dD", (D,), False),
        _ptr(g["dz"], "dz", (M, D), False), _ptr(g["dh0"], "dh0", (batch, D, N), False),
        wp, wn, _stream(stream)))
    return g


def selective_scan_backward_noalloc(u, delta, A_log, B, C, D_vec, z, h0, dout, *, batch,
                                    seq_len, disc, need_dh0=False, out=None, stream=None,
                                    exact=False, h_ckpt=None):
    """``selective_scan_backward`` through the entry point whose workspace is the
    library's static scratch array (for callers that cannot allocate; at most
    NOALLOC_SCRATCH_BYTES of workspace; calls overlapping on one GPU race).
    ``out``: optional dict of preallocated gradient tensors (the keys of the
    result), so that the call itself allocates nothing."""
    D, N = A_log.shape
    M = batch * seq_len
    shapes = {"du": (M, D), "ddelta": (M, D), "dA_log": (D, N), "dB": (M, N), "dC": (M, N),
              "dD": (D,), "dz": (M, D), "dh0": (batch, D, N)}
    want = {"du": True, "ddelta": True, "dA_log": True, "dB": True, "dC": True,
            "dD": D_vec is not None, "dz": z is not None, "dh0": need_dh0}
    out = dict(out or {})
    g = {k: (out[k] if k in out else _empty(shapes[k], u)) if want[k] else None for k in shapes}
    dims = make_dims(batch, seq_len, D, N, 1, exact, h_ckpt is not None)
    _check("mss_selective_scan_backward_noalloc", lib().mss_selective_scan_backward_noalloc(
        ctypes.byref(dims), _disc(disc), _ptr(u, "u", (M, D)), _ptr(delta, "delta", (M, D)),
        _ptr(A_log, "A_log", (D, N)), _ptr(B, "B", (M, N)), _ptr(C, "C", (M, N)),
        _ptr(D_vec, "D_vec", (D,), False), _ptr(z, "z", (M, D), False),
        _ptr(h0, "h0", (batch, D, N), False),
        _ptr(h_ckpt, "h_ckpt", (batch, ckpt_steps(seq_len), D, N), False),
        _ptr(dout, "dout", (M, D)),
        _ptr(g["du"], "du", (M, D)), _ptr(g["ddelta"], "ddelta", (M, D)),
        _ptr(g["dA_log"], "dA_log", (D, N)), _ptr(g["dB"], "dB", (M, N)),
        _ptr(g["dC"], "dC", (M, N)), _ptr(g["dD"], "dD", (D,), False),
        _ptr(g["dz"], "dz", (M, D), False), _ptr(g["dh0"], "dh0", (batch, D, N), False),
        _stream(stream)))
    return g


def conv1d_silu_backward(x, w_conv, b_conv, du, *, batch, seq_len, workspace=None, stream=None):
    """Gradients of ``conv1d_silu`` against ``du``: (dx, dw_conv, db_conv)."""
    D, K = w_conv.shape
    M = batch * seq_len
    dx, dw, db = _empty((M, D), x), _empty((D, K), x), _empty((D,), x)
    wp, wn, _keep = _workspace(OP_CONV1D_SILU_BACKWARD, x, workspace, stream, batch=batch,
                               seq_len=seq_len, d_inner=D, d_state=1, d_conv=K)
    dims = make_dims(batch, seq_len, D, 1, K)
    _check("mss_conv1d_silu_backward", lib().mss_conv1d_silu_backward(
        ctypes.byref(dims), _ptr(x, "x", (M, D)), _ptr(w_conv, "w_conv", (D, K)),
        _ptr(b_conv, "b_conv", (D,), False), _ptr(du, "du", (M, D)), _ptr(dx, "dx", (M, D)),
        _ptr(dw, "dw_conv", (D, K)), _ptr(db, "db_conv", (D,)), wp, wn, _stream(stream)))
    return dx, dw, db


def ssd_scan(x, dt, A_log, B, C, D_vec=None, dt_bias=None, h0=None, *, batch, seq_len,
             head_dim, d_state, n_groups=1, disc, h_last=False, out=None, stream=None,
             exact=False):
    """Mamba-2 SSD scan: y (batch*seq_len, H*head_dim) and, when ``h_last`` is
    True (or a tensor), the final state (batch, H, head_dim, d_state).
    ``exact``: no time split."""
    H = A_log.shape[0]
    P, N, G = head_dim, d_state, n_groups
    M = batch * seq_len
    y = out if out is not None else _empty((M, H * P), x)
    hl = (h_last if not isinstance(h_last, bool) else
          (_empty((batch, H, P, N), x) if h_last else None))
    dims = make_ssd_dims(batch, seq_len, H, P, N, G, exact)
    _check("mss_ssd_scan", lib().mss_ssd_scan(
        ctypes.byref(dims), _disc(disc), _ptr(x, "x", (M, H * P)), _ptr(dt, "dt", (M, H)),
        _ptr(A_log, "A_log", (H,)), _ptr(B, "B", (M, G * N)), _ptr(C, "C", (M, G * N)),
        _ptr(D_vec, "D_vec", (H,), False), _ptr(dt_bias, "dt_bias", (H,), False),
        _ptr(h0, "h0", (batch, H, P, N), False), _ptr(y, "y", (M, H * P)),
        _ptr(hl, "h_last", (batch, H, P, N), False), _stream(stream)))
    return y, hl
