"""C-ABI checks that need no GPU: the library loads, exports every function
include/mss.h declares, and rejects bad arguments before any launch.

Pointers here are fake aligned integers: validation never dereferences them,
and every call below fails (or is empty) before reaching a kernel launch."""
import ctypes
import os
import re

import pytest

import mamba_selective_scan_causal_amd as mss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mss.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(mss_\w+)\s*\(", text, re.M)))


def header_define(name):
    m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)\)?", open(HEADER).read())
    return int(m.group(1))


@pytest.fixture(scope="module")
def L():
    return mss.lib()


def test_exports_every_declared_function(L):
    fns = header_functions()
    assert set(fns) == set(mss.EXPORTS), fns
    for f in fns:
        assert hasattr(L, f), f"{f} not exported"


def test_version_and_strerror(L):
    assert L.mss_version() == header_define("MSS_VERSION")
    for name in ("MSS_OK", "MSS_EINVAL", "MSS_EALIGN", "MSS_EALIAS", "MSS_EWORKSPACE",
                 "MSS_EHIP"):
        s = L.mss_strerror(header_define(name))
        assert s and s != b"unknown status"
    assert L.mss_strerror(12345) == b"unknown status"
    assert ctypes.sizeof(mss.Dims) == 48


EINVAL, EALIGN, EALIAS = (header_define(n) for n in ("MSS_EINVAL", "MSS_EALIGN", "MSS_EALIAS"))
BASE = 0x7F0000000000


def fake(i, nbytes=1 << 20):
    """Distinct, 16-byte aligned, non-overlapping fake device addresses."""
    return ctypes.c_void_p(BASE + i * (1 << 32))


def scan_call(L, dims, disc=0, **over):
    args = dict(u=fake(1), delta=fake(2), A_log=fake(3), B=fake(4), C=fake(5), D_vec=fake(6),
                z=fake(7), h0=None, y=fake(8), h_cache=None, h_last=None)
    args.update(over)
    return L.mss_selective_scan(ctypes.byref(dims), disc, *args.values(), None)


def test_scan_validation(L):
    d = mss.make_dims(2, 16, 64, 16, 4)
    assert L.mss_selective_scan(None, 0, *([None] * 11), None) == EINVAL
    bad = mss.make_dims(2, 16, 64, 16, 4)
    bad.struct_size = 40
    assert scan_call(L, bad) == EINVAL
    bad = mss.make_dims(2, 16, 64, 16, 4)
    bad.flags = 4                                                         # unknown flag bit
    assert scan_call(L, bad) == EINVAL
    bad.flags = -1
    assert scan_call(L, bad) == EINVAL
    assert scan_call(L, mss.make_dims(2, 16, 64, 17, 4)) == EINVAL       # N > 16
    assert scan_call(L, mss.make_dims(2, 16, 64, 0, 4)) == EINVAL        # N < 1
    assert scan_call(L, mss.make_dims(-1, 16, 64, 16, 4)) == EINVAL      # negative size
    assert scan_call(L, d, disc=2) == EINVAL                              # disc has no default
    assert scan_call(L, d, u=None) == EINVAL                              # required tensor
    assert scan_call(L, d, C=None) == EINVAL
    assert scan_call(L, d, delta=ctypes.c_void_p(BASE + 4)) == EALIGN
    assert scan_call(L, d, y=fake(1)) == EALIAS                           # y == u
    assert scan_call(L, d, y=ctypes.c_void_p(BASE + 2 * (1 << 32) + 256)) == EALIAS  # y inside delta
    assert scan_call(L, d, h_last=fake(8)) == EALIAS                      # two outputs overlap
    huge = mss.make_dims(1 << 40, 1 << 20, 1 << 20, 16, 4)
    assert scan_call(L, huge) == EINVAL                                   # overflowing sizes


def test_empty_problems_launch_nothing(L):
    # zero channels: nothing to compute; only B and C (M, N) still hold elements
    dims = mss.make_dims(2, 16, 0, 16, 4)
    assert L.mss_selective_scan(ctypes.byref(dims), 0, *([None] * 11), None) == EINVAL
    scan = [None] * 11
    scan[3], scan[4] = fake(4), fake(5)
    assert L.mss_selective_scan(ctypes.byref(dims), 0, *scan, None) == 0
    core = [None] * 13
    core[5], core[6] = fake(4), fake(5)
    assert L.mss_mamba1_core(ctypes.byref(dims), 1, *core, None) == 0
    assert L.mss_conv1d_silu(ctypes.byref(dims), None, None, None, None, None) == 0
    step = [None] * 12
    step[4], step[5] = fake(4), fake(5)
    assert L.mss_selective_step(ctypes.byref(dims), 0, *step, None) == 0
    # zero batch: the per-channel parameters still hold elements and are required
    dims = mss.make_dims(0, 16, 64, 16, 4)
    assert L.mss_selective_scan(ctypes.byref(dims), 0, *([None] * 11), None) == EINVAL
    assert L.mss_selective_scan(ctypes.byref(dims), 0, None, None, fake(3), *([None] * 8),
                                None) == 0
    core = [None] * 13
    core[1], core[4] = fake(2), fake(3)   # w_conv, A_log
    assert L.mss_mamba1_core(ctypes.byref(dims), 1, *core, None) == 0
    assert L.mss_conv1d_silu(ctypes.byref(dims), None, fake(2), None, None, None) == 0
    step = [None] * 12
    step[3], step[7] = fake(3), fake(4)   # A_log, w_conv
    assert L.mss_selective_step(ctypes.byref(dims), 0, *step, None) == 0
    # seq_len 0 without h_last: nothing to launch
    dims = mss.make_dims(2, 0, 64, 16, 4)
    assert L.mss_selective_scan(ctypes.byref(dims), 0, None, None, fake(3), None, None, None, None,
                                None, None, None, None, None) == 0


def test_core_and_conv_validation(L):
    d = mss.make_dims(2, 16, 64, 16, 9)  # K > 8
    assert L.mss_conv1d_silu(ctypes.byref(d), fake(1), fake(2), None, fake(3), None) == EINVAL
    d = mss.make_dims(2, 16, 64, 16, 4)
    assert L.mss_conv1d_silu(ctypes.byref(d), fake(1), fake(2), None, fake(1), None) == EALIAS
    assert L.mss_conv1d_silu(ctypes.byref(d), fake(1), None, None, fake(3), None) == EINVAL
    args = [fake(i) for i in range(1, 14)]
    args[1] = None  # w_conv missing
    assert L.mss_mamba1_core(ctypes.byref(d), 0, *args, None) == EINVAL
    d0 = mss.make_dims(2, 16, 64, 16, 0)  # K = 0
    assert L.mss_mamba1_core(ctypes.byref(d0), 0, *[fake(i) for i in range(1, 14)], None) == EINVAL
    # an empty sequence does not excuse a d_inner whose (D, K) conv weight
    # size overflows
    wide = mss.make_dims(1, 0, 1 << 62, 1, 4)
    assert L.mss_conv1d_silu(ctypes.byref(wide), fake(1), fake(2), None, fake(3), None) == EINVAL
    assert L.mss_mamba1_core(ctypes.byref(wide), 0, *[fake(i) for i in range(1, 14)],
                             None) == EINVAL
    assert L.mss_selective_step(ctypes.byref(mss.make_dims(0, 1, 1 << 62, 1, 4)), 0,
                                *[fake(i) for i in range(1, 13)], None) == EINVAL
    assert conv_bwd_call(L, wide, ws_size=0) == EINVAL


def test_step_validation(L):
    d = mss.make_dims(4, 1, 64, 16, 4)
    args = [fake(i) for i in range(1, 13)]  # x z delta A_log B C D_vec w b conv_state h y
    a = list(args)
    a[9] = None  # conv_state required when K > 1
    assert L.mss_selective_step(ctypes.byref(d), 0, *a, None) == EINVAL
    a = list(args)
    a[11] = a[0]  # y == x
    assert L.mss_selective_step(ctypes.byref(d), 0, *a, None) == EALIAS
    a = list(args)
    a[10] = ctypes.c_void_p(BASE + 8)
    assert L.mss_selective_step(ctypes.byref(d), 0, *a, None) == EALIGN
    assert L.mss_selective_step(ctypes.byref(d), 5, *args, None) == EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mss, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mss, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        mss.lib()


def core_strided(L, dims, strides, **over):
    args = dict(x=fake(1), w_conv=fake(2), b_conv=None, delta=fake(3), A_log=fake(4), B=fake(5),
                C=fake(6), D_vec=fake(7), z=fake(8), h0=None, y=fake(9), h_cache=None,
                h_last=None)
    args.update(over)
    s = ctypes.byref(strides) if strides is not None else None
    return L.mss_mamba1_core_strided(ctypes.byref(dims), s, 0, *args.values(), None)


def test_strided_validation(L):
    d = mss.make_dims(2, 16, 64, 16, 4)
    ok = mss.make_strides(128, 128, 64, 48, 48, 64)
    assert core_strided(L, d, None) == EINVAL
    bad = mss.make_strides(128, 128, 64, 48, 48, 64)
    bad.struct_size = 8
    assert core_strided(L, d, bad) == EINVAL
    for field, width in (("x", 64), ("z", 64), ("delta", 64), ("B", 16), ("C", 16), ("y", 64)):
        s = mss.make_strides(128, 128, 64, 48, 48, 64)
        setattr(s, field, width - 1)               # row stride below the row width
        assert core_strided(L, d, s) == EINVAL, field
    # activations may be 4-byte aligned in the strided call: the call gets past
    # the alignment checks and is rejected only for y overlapping x
    x4 = ctypes.c_void_p(BASE + 1 * (1 << 32) + 4)
    assert core_strided(L, d, ok, x=x4, y=ctypes.c_void_p(BASE + (1 << 32) + 64)) == EALIAS
    # the dense call keeps the 16-byte rule for the same pointer
    dense = [x4, fake(2), None, fake(3), fake(4), fake(5), fake(6), fake(7), fake(8), None,
             fake(9), None, None]
    assert L.mss_mamba1_core(ctypes.byref(d), 0, *dense, None) == EALIGN
    # state tensors keep the 16-byte rule in the strided call
    assert core_strided(L, d, ok, h0=ctypes.c_void_p(BASE + 10 * (1 << 32) + 8)) == EALIGN
    # x and z as interleaved halves of one (M, 2D) buffer are fine (both inputs);
    # y inside that buffer's span is not
    xz = BASE + 11 * (1 << 32)
    s = mss.make_strides(128, 128, 64, 48, 48, 64)
    assert core_strided(L, d, s, x=ctypes.c_void_p(xz), z=ctypes.c_void_p(xz + 256),
                        y=ctypes.c_void_p(xz + 128 * 4 * 5)) == EALIAS
    # empty problem: nothing to launch
    d0 = mss.make_dims(2, 16, 0, 16, 4)
    assert L.mss_selective_scan_strided(ctypes.byref(d0), ctypes.byref(ok), 1, None, None, None,
                                        fake(5), fake(6), None, None, None, None, None, None,
                                        None) == 0


EWORKSPACE = header_define("MSS_EWORKSPACE")
OP_SCAN_BWD = header_define("MSS_OP_SELECTIVE_SCAN_BACKWARD")
OP_CONV_BWD = header_define("MSS_OP_CONV1D_SILU_BACKWARD")


def ws_bytes(L, dims, op):
    n = ctypes.c_size_t(123)
    st = L.mss_workspace_bytes(ctypes.byref(dims) if dims is not None else None, op,
                               ctypes.byref(n))
    return st, n.value


def test_workspace_query(L):
    assert (OP_SCAN_BWD, OP_CONV_BWD) == (mss.OP_SELECTIVE_SCAN_BACKWARD,
                                          mss.OP_CONV1D_SILU_BACKWARD)
    d = mss.make_dims(2, 512, 256, 16, 4)
    st, n = ws_bytes(L, d, OP_SCAN_BWD)
    # at least the checkpoints (8 floats per lane and block, 2 lanes per
    # channel) and the per-tile dB / dC rows
    assert st == 0 and n >= 2 * 512 * 256 * 2 * 4 + 2 * (2 * 8 * 512 * 16 * 4) and n % 256 == 0
    st, n = ws_bytes(L, d, OP_CONV_BWD)
    assert st == 0 and n > 0 and n % 256 == 0
    assert ws_bytes(L, mss.make_dims(0, 512, 256, 16, 4), OP_SCAN_BWD) == (0, 0)
    assert ws_bytes(L, mss.make_dims(2, 0, 256, 16, 4), OP_CONV_BWD) == (0, 0)
    assert ws_bytes(L, d, 99)[0] == EINVAL
    assert ws_bytes(L, None, OP_SCAN_BWD)[0] == EINVAL
    assert ws_bytes(L, mss.make_dims(2, 512, 256, 17, 4), OP_SCAN_BWD)[0] == EINVAL
    assert ws_bytes(L, mss.make_dims(2, 512, 256, 16, 9), OP_CONV_BWD)[0] == EINVAL
    assert L.mss_workspace_bytes(ctypes.byref(d), OP_SCAN_BWD, None) == EINVAL


def scan_bwd_call(L, dims, disc=0, ws_size=None, **over):
    args = dict(u=fake(1), delta=fake(2), A_log=fake(3), B=fake(4), C=fake(5), D_vec=fake(6),
                z=fake(7), h0=None, h_ckpt=None, dout=fake(8), du=fake(9), ddelta=fake(10),
                dA_log=fake(11), dB=fake(12), dC=fake(13), dD=fake(14), dz=fake(15), dh0=None,
                ws=fake(16))
    args.update(over)
    if ws_size is None:
        ws_size = ws_bytes(L, dims, OP_SCAN_BWD)[1]
    vals = list(args.values())
    return L.mss_selective_scan_backward(ctypes.byref(dims), disc, *vals, ws_size, None)


def test_scan_backward_validation(L):
    d = mss.make_dims(2, 64, 64, 16, 4)
    assert scan_bwd_call(L, d, disc=3) == EINVAL
    for name in ("u", "delta", "A_log", "B", "C", "dout", "du", "ddelta", "dA_log", "dB", "dC"):
        assert scan_bwd_call(L, d, **{name: None}) == EINVAL, name
    assert scan_bwd_call(L, d, dz=None) == EINVAL                 # z given needs dz
    assert scan_bwd_call(L, d, dout=ctypes.c_void_p(BASE + 8 * (1 << 32) + 4)) == EALIGN
    assert scan_bwd_call(L, d, du=fake(1)) == EALIAS              # output on an input
    assert scan_bwd_call(L, d, dB=fake(12), dC=fake(12)) == EALIAS
    assert scan_bwd_call(L, d, ws=fake(9)) == EALIAS              # workspace on an output
    assert scan_bwd_call(L, d, ws=None) == EWORKSPACE
    need = ws_bytes(L, d, OP_SCAN_BWD)[1]
    assert scan_bwd_call(L, d, ws_size=need - 1) == EWORKSPACE
    assert scan_bwd_call(L, d, ws=ctypes.c_void_p(BASE + 16 * (1 << 32) + 16)) == EALIGN
    # checkpoints from the forward: the flag and the pointer go together, the
    # checkpoints are an input (no output may overlap them), and they shrink
    # the workspace
    dck = mss.make_dims(2, 64, 64, 16, 4, ckpt8=True)
    need_ck = ws_bytes(L, dck, OP_SCAN_BWD)[1]
    assert 0 < need_ck < need
    assert scan_bwd_call(L, dck, ws_size=need_ck) == EINVAL              # flag without h_ckpt
    assert scan_bwd_call(L, d, h_ckpt=fake(17)) == EINVAL                # h_ckpt without flag
    assert scan_bwd_call(L, dck, h_ckpt=fake(17), ws_size=need_ck - 1) == EWORKSPACE
    assert scan_bwd_call(L, dck, h_ckpt=fake(9), ws_size=need_ck) == EALIAS   # du on h_ckpt


def conv_bwd_call(L, dims, ws_size=None, **over):
    args = dict(x=fake(1), w=fake(2), b=fake(3), du=fake(4), dx=fake(5), dw=fake(6), db=fake(7),
                ws=fake(8))
    args.update(over)
    if ws_size is None:
        ws_size = ws_bytes(L, dims, OP_CONV_BWD)[1]
    return L.mss_conv1d_silu_backward(ctypes.byref(dims), *args.values(), ws_size, None)


def test_conv_backward_validation(L):
    d = mss.make_dims(2, 64, 64, 1, 4)
    for name in ("x", "w", "du", "dx", "dw"):
        assert conv_bwd_call(L, d, **{name: None}) == EINVAL, name
    assert conv_bwd_call(L, mss.make_dims(2, 64, 64, 1, 0)) == EINVAL
    assert conv_bwd_call(L, d, dx=fake(1)) == EALIAS
    assert conv_bwd_call(L, d, ws=None) == EWORKSPACE
    assert conv_bwd_call(L, d, ws_size=1) == EWORKSPACE
    assert conv_bwd_call(L, d, du=ctypes.c_void_p(BASE + 4 * (1 << 32) + 8)) == EALIGN


def ssd_call(L, dims, **over):
    args = dict(x=fake(1), dt=fake(2), A_log=fake(3), B=fake(4), C=fake(5), D=fake(6),
                bias=fake(7), h0=None, y=fake(8), h_last=None)
    args.update(over)
    disc = args.pop("disc", 1)
    return L.mss_ssd_scan(ctypes.byref(dims) if dims is not None else None, disc,
                          *args.values(), None)


def test_ssd_validation(L):
    d = mss.make_ssd_dims(2, 64, 8, 64, 128, 2)
    assert ssd_call(L, None) == EINVAL
    bad = mss.make_ssd_dims(2, 64, 8, 64, 128, 2)
    bad.struct_size = 48
    assert ssd_call(L, bad) == EINVAL
    assert ssd_call(L, mss.make_ssd_dims(2, 64, 8, 48, 128)) == EINVAL     # head_dim
    assert ssd_call(L, mss.make_ssd_dims(2, 64, 8, 64, 96)) == EINVAL      # d_state
    assert ssd_call(L, mss.make_ssd_dims(2, 64, 8, 64, 128, 3)) == EINVAL  # G does not divide H
    assert ssd_call(L, mss.make_ssd_dims(2, 64, 0, 64, 128)) == EINVAL
    assert ssd_call(L, d, disc=2) == EINVAL
    for name in ("x", "dt", "A_log", "B", "C", "y"):
        assert ssd_call(L, d, **{name: None}) == EINVAL, name
    assert ssd_call(L, d, y=fake(1)) == EALIAS
    assert ssd_call(L, d, x=ctypes.c_void_p(BASE + (1 << 32) + 8)) == EALIGN
    assert ssd_call(L, mss.make_ssd_dims(0, 64, 8, 64, 128, 2)) == 0        # empty: nothing to do
    assert ctypes.sizeof(mss.SsdDims) == 56


def test_binding_loads_libmss_on_torchs_hip_runtime():
    """libmss must resolve libamdhip64.so.7 to the runtime torch loaded: a
    fresh process that asks the binding for the library (before importing
    torch itself) ends up with one HIP runtime mapped, torch's."""
    import subprocess
    import sys
    code = ("import mamba_selective_scan_causal_amd as m; m.lib(); "
            "maps = [l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l]; "
            "print(sorted(set(maps)))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))), timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert len(libs) == 1 and "torch" in libs[0], libs


def test_noalloc_backward_refuses_past_its_scratch(L):
    """The allocation-free scan backward checks its size against the static
    scratch array before any HIP call, so on a machine without a GPU a
    request past MSS_NOALLOC_SCRATCH_BYTES comes back as MSS_ESCRATCH; bad
    arguments are still reported first."""
    assert re.search(r"#define MSS_NOALLOC_SCRATCH_BYTES \(256ull << 20\)", open(HEADER).read())
    assert mss.NOALLOC_SCRATCH_BYTES == 256 << 20
    assert header_define("MSS_ESCRATCH") == mss.MSS_ESCRATCH
    d = mss.make_dims(8, 2048, 1536, 16, 4)
    assert ws_bytes(L, d, OP_SCAN_BWD)[1] > mss.NOALLOC_SCRATCH_BYTES

    def call(dims, disc=0, **over):
        args = dict(u=fake(1), delta=fake(2), A_log=fake(3), B=fake(4), C=fake(5),
                    D_vec=fake(6), z=fake(7), h0=None, h_ckpt=None, dout=fake(8), du=fake(9),
                    ddelta=fake(10), dA_log=fake(11), dB=fake(12), dC=fake(13), dD=fake(14),
                    dz=fake(15), dh0=None)
        args.update(over)
        return L.mss_selective_scan_backward_noalloc(ctypes.byref(dims), disc,
                                                     *args.values(), None)

    assert call(d) == mss.MSS_ESCRATCH
    assert call(d, disc=3) == EINVAL
    assert call(d, du=fake(1)) == EALIAS
    assert call(d, dout=None) == EINVAL
    assert b"static" in L.mss_strerror(mss.MSS_ESCRATCH)
