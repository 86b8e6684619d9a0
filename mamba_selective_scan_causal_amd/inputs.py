"""Seeded synthetic inputs for the Mamba-1 (S6) block core.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic (no convolution, activation, discretisation or scan).
It is the one piece shared by the HIP path's tests/benchmark and the CPU
oracle, so both always see bit-identical fp32 inputs.

Tensor layouts follow the Mamba-1 CPU mirror's layout note
(builderforce-memory-engine 2026.7.12 -> 2026.9.27, src/training/mamba1_cpu.ts,
file header): activations are (M, D) row-major with M = batch * seq_len and
row r = b * seq_len + t; B and C are (M, N); A_log is (D, N); wConv is (D, K)
depthwise; hCache is (B, L, D, N).

Distribution notation: ``N(mu, v)`` takes v as the *variance*.  Every tensor
gets its own child of ``SeedSequence(SEED_BASE + seed_index)`` in a fixed
order, and large tensors are drawn in fixed-size blocks, each block from its
own grandchild stream, so the result does not depend on thread count.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_BASE = 0x5EED0000
_BLOCK = 1 << 22  # elements per independently seeded block

# Fixed spawn order of the per-tensor child streams.
_STREAMS = ("x", "z", "delta", "B", "C", "alog_mask", "alog_choice",
            "w_conv", "D_vec", "h0", "conv_state", "b_conv")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload.

    ``mode == "sequence"``: one causal pass over ``seq_len`` steps.
    ``mode == "step"``: ``seq_len`` consecutive single-token recurrent steps
    with a carried state (h, conv_state) drawn at random.
    """
    name: str
    batch: int
    seq_len: int
    d_inner: int
    d_state: int = 16
    d_conv: int = 4
    mode: str = "sequence"
    delta_mean: float = -1.0
    delta_var: float = 1.0
    alog_clamp_frac: float = 0.0      # fraction of A_log entries replaced by -12 or 6
    d_vec: str = "uniform"            # "ones" -> 1, "uniform" -> U(0.5, 1.5)
    b_conv: str = "zero"              # "zero" or "normal" (N(0, 1/4))
    h0: bool = False                  # sequence mode: draw an initial state
    hcache: bool = False              # whether the workload emits the per-step state cache
    h_var: float = 0.1                # step mode: carried state ~ N(0, h_var)
    seed_index: int = 0

    @property
    def M(self) -> int:
        return self.batch * self.seq_len

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is exercised on.  Sizes are those of a
# 130M-class (d_inner 1536) and a 2.8B-class (d_inner 5120) Mamba-1 block.
TINY_CLAMP = Workload("b1_l64_d32_n16_k4_clamp", 1, 64, 32, delta_mean=-1.0, delta_var=1.0,
                      alog_clamp_frac=0.1, d_vec="ones", hcache=True, seed_index=0)
SMALL = Workload("b2_l512_d256_n16_k4", 2, 512, 256, delta_mean=-1.0, delta_var=1.0,
                 d_vec="uniform", hcache=True, seed_index=1)
MAMBA_130M = Workload("b8_l2048_d1536_n16_k4", 8, 2048, 1536, delta_mean=-2.0, delta_var=0.5,
                      seed_index=2)
MAMBA_2P8B = Workload("b4_l8192_d5120_n16_k4", 4, 8192, 5120, delta_mean=-2.0, delta_var=0.5,
                      seed_index=3)
DECODE = Workload("decode_b256_d5120_n16_k4_x64", 256, 64, 5120, mode="step",
                  delta_mean=-2.0, delta_var=0.5, h_var=0.1, seed_index=4)

WORKLOADS = {w.name: w for w in (TINY_CLAMP, SMALL, MAMBA_130M, MAMBA_2P8B, DECODE)}


def _children(w: Workload, seed_offset: int):
    ss = np.random.SeedSequence(SEED_BASE + w.seed_index + 1000 * seed_offset)
    return dict(zip(_STREAMS, ss.spawn(len(_STREAMS))))


def _normal(seq: np.random.SeedSequence, shape, mean: float, var: float,
            threads: int = 8) -> np.ndarray:
    """fp32 normal draws, generated block-wise from per-block child streams."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nblk = max(1, math.ceil(n / _BLOCK))
    seqs = seq.spawn(nblk)
    sd = np.float32(math.sqrt(var))
    mu = np.float32(mean)

    def fill(i):
        lo, hi = i * _BLOCK, min(n, (i + 1) * _BLOCK)
        g = np.random.Generator(np.random.PCG64(seqs[i]))
        blk = g.standard_normal(hi - lo, dtype=np.float32)
        blk *= sd
        blk += mu
        out[lo:hi] = blk

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _uniform(seq, shape, lo, hi):
    g = np.random.Generator(np.random.PCG64(seq))
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def _a_log(w: Workload, ch) -> np.ndarray:
    # S4D-real initialisation: A_log[d, n] = log(n + 1), n counted from 0.
    base = np.log(np.arange(1, w.d_state + 1, dtype=np.float64))
    a = np.broadcast_to(base, (w.d_inner, w.d_state)).copy()
    if w.alog_clamp_frac > 0:
        gm = np.random.Generator(np.random.PCG64(ch["alog_mask"]))
        gc = np.random.Generator(np.random.PCG64(ch["alog_choice"]))
        mask = gm.random(a.shape) < w.alog_clamp_frac
        choice = np.where(gc.random(a.shape) < 0.5, -12.0, 6.0)
        a = np.where(mask, choice, a)
    return a.astype(np.float32)


def generate(w: Workload, seed_offset: int = 0, threads: int = 8) -> dict:
    """Draw every input tensor of workload ``w`` (all fp32, C-contiguous)."""
    ch = _children(w, seed_offset)
    D, N, K = w.d_inner, w.d_state, w.d_conv
    out = {}
    if w.mode == "sequence":
        act = (w.M, D)
        row = (w.M, N)
    elif w.mode == "step":
        act = (w.seq_len, w.batch, D)
        row = (w.seq_len, w.batch, N)
    else:
        raise ValueError(f"unknown mode {w.mode!r}")
    out["x"] = _normal(ch["x"], act, 0.0, 1.0, threads)
    out["z"] = _normal(ch["z"], act, 0.0, 1.0, threads)
    out["delta"] = _normal(ch["delta"], act, w.delta_mean, w.delta_var, threads)
    out["B"] = _normal(ch["B"], row, 0.0, 1.0, threads)
    out["C"] = _normal(ch["C"], row, 0.0, 1.0, threads)
    out["A_log"] = _a_log(w, ch)
    out["w_conv"] = _normal(ch["w_conv"], (D, K), 0.0, 0.25)
    if w.b_conv == "normal":
        out["b_conv"] = _normal(ch["b_conv"], (D,), 0.0, 0.25)
    else:
        out["b_conv"] = np.zeros(D, dtype=np.float32)
    if w.d_vec == "ones":
        out["D_vec"] = np.ones(D, dtype=np.float32)
    else:
        out["D_vec"] = _uniform(ch["D_vec"], (D,), 0.5, 1.5)
    if w.mode == "step":
        out["h"] = _normal(ch["h0"], (w.batch, D, N), 0.0, w.h_var, threads)
        out["conv_state"] = _normal(ch["conv_state"], (w.batch, max(K - 1, 0), D), 0.0, 1.0)
    elif w.h0:
        out["h0"] = _normal(ch["h0"], (w.batch, D, N), 0.0, w.h_var, threads)
    return out


def cotangent(w: Workload, seed_offset: int = 0, threads: int = 8) -> np.ndarray:
    """A seeded N(0, 1) gradient of the output (M, D) for the backward passes,
    from a stream of its own (the inputs of ``generate`` are unchanged)."""
    seq = np.random.SeedSequence([SEED_BASE + w.seed_index + 1000 * seed_offset, 0xD07])
    return _normal(seq, (w.M, w.d_inner), 0.0, 1.0, threads)


@dataclasses.dataclass(frozen=True)
class SsdWorkload:
    """Shape and value recipe of a Mamba-2 SSD scan workload: H heads of P
    channels, G groups of N states.  x ~ N(0, 1); raw dt ~ N(dt_mean, dt_var)
    per (row, head); A_log = log(U[1, 16]) per head; B, C ~ N(0, 1);
    D ~ U(0.5, 1.5); dt_bias = 0; optional h0 ~ N(0, 0.1)."""
    name: str
    batch: int
    seq_len: int
    n_heads: int
    head_dim: int
    d_state: int
    n_groups: int = 1
    dt_mean: float = -2.0
    dt_var: float = 0.5
    h0: bool = False
    seed_index: int = 20

    @property
    def M(self) -> int:
        return self.batch * self.seq_len

    def with_(self, **kw) -> "SsdWorkload":
        return dataclasses.replace(self, **kw)


SSD_TINY = SsdWorkload("ssd_b1_l100_h4_p16_n32_g2", 1, 100, 4, 16, 32, n_groups=2, h0=True,
                       seed_index=21)
SSD_SMALL = SsdWorkload("ssd_b2_l512_h8_p64_n128_g1", 2, 512, 8, 64, 128, h0=True,
                        seed_index=22)
SSD_2P7B = SsdWorkload("ssd_b4_l8192_h80_p64_n128_g1", 4, 8192, 80, 64, 128, seed_index=23)

_SSD_STREAMS = ("x", "dt", "A_log", "B", "C", "D_vec", "h0")


def generate_ssd(w: SsdWorkload, seed_offset: int = 0, threads: int = 8) -> dict:
    """Draw every input of SSD workload ``w`` (fp32, C-contiguous)."""
    ss = np.random.SeedSequence([SEED_BASE + w.seed_index + 1000 * seed_offset, 0x55D])
    ch = dict(zip(_SSD_STREAMS, ss.spawn(len(_SSD_STREAMS))))
    H, P, N, G = w.n_heads, w.head_dim, w.d_state, w.n_groups
    out = {
        "x": _normal(ch["x"], (w.M, H * P), 0.0, 1.0, threads),
        "dt": _normal(ch["dt"], (w.M, H), w.dt_mean, w.dt_var, threads),
        "A_log": np.log(_uniform(ch["A_log"], (H,), 1.0, 16.0)).astype(np.float32),
        "B": _normal(ch["B"], (w.M, G * N), 0.0, 1.0, threads),
        "C": _normal(ch["C"], (w.M, G * N), 0.0, 1.0, threads),
        "D_vec": _uniform(ch["D_vec"], (H,), 0.5, 1.5),
        "dt_bias": np.zeros(H, dtype=np.float32),
    }
    if w.h0:
        out["h0"] = _normal(ch["h0"], (w.batch, H, P, N), 0.0, 0.1, threads)
    return out
