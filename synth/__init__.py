"""Seeded synthetic inputs for the selective scan and the SSD chunked form.

Used by the GPU parity tests, by ``bench.py`` and by the CPU oracle's tests.
This module draws numbers and rounds them to storage types; it computes no
part of the scan itself.  Every value is a pure function of
(seed, stream id, flat index) -- see ``synth.c`` -- so any slice can be
regenerated independently.

bf16 tensors are returned as ``numpy.uint16`` bit patterns; fp32 as float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

NORMAL, UNIFORM, SOFTPLUS_NORMAL, NEG_EXP_UNIFORM, NEG_IDX, CONST = range(6)

# Stream ids: one per tensor role, so tensors never share random numbers.
STREAM = {"x": 1, "delta": 2, "A": 3, "B": 4, "C": 5, "D": 6, "z": 7, "h0": 8, "delta_bias": 9, "conv_w": 10,
          "conv_b": 11, "w_in": 12, "w_x": 13, "w_dt": 14, "w_out": 15, "u": 16}


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_int64, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_int]
        lib.synth_raw.restype = None
        lib.synth_raw.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_f32_to_bf16.restype = ctypes.c_uint16
        lib.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass(frozen=True)
class Dist:
    kind: int
    p0: float = 0.0
    p1: float = 1.0
    period: int = 1


def fill(shape, dist: Dist, dtype: str, seed: int, stream: int, start: int = 0) -> np.ndarray:
    """Elements start..start+prod(shape) of a stream, reshaped.  dtype: 'f32' or 'bf16'."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if n:
        _load().synth_fill(out.ctypes.data, n, start, 1 if dtype == "bf16" else 0, dist.kind, dist.p0, dist.p1,
                           dist.period, seed, stream, _threads())
    return out.reshape(shape)


def raw(n: int, start: int, seed: int, stream: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_raw(out.ctypes.data, n, start, seed, stream)
    return out


def f32_to_bf16_bits(v: float) -> int:
    return int(_load().synth_f32_to_bf16(float(v)))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else a.astype(np.float64)


# --------------------------------------------------------------------------
# Workload recipes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class ScanSpec:
    """Selective scan problem: x, delta, z, y (batch, L, D); B, C (batch, L, N);
    A (D, N); D (D)."""
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io: str  # 'f32' or 'bf16'
    has_z: bool
    has_D: bool
    A: Dist
    delta: Dist
    euler: bool = False
    x: Dist = Dist(NORMAL, 0.0, 1.0)
    B: Dist = Dist(NORMAL, 0.0, 1.0)
    C: Dist = Dist(NORMAL, 0.0, 1.0)
    z: Dist = Dist(NORMAL, 0.0, 1.0)
    Dskip: Dist = Dist(NORMAL, 0.0, 1.0)

    @property
    def tc(self) -> int:
        return self.batch * self.seqlen * self.dim

    def algorithmic_bytes(self) -> int:
        """Each input read once, y written once; B and C once per token."""
        e = 2 if self.io == "bf16" else 4
        per_tc = e * (3 + (1 if self.has_z else 0))  # x, delta, [z], y
        per_tok = 2 * self.dstate * e  # B, C
        return self.tc * per_tc + self.batch * self.seqlen * per_tok + self.dim * self.dstate * 4 + \
            (self.dim * 4 if self.has_D else 0)


@dataclass(frozen=True)
class ConvSpec:
    """Causal depthwise convolution: x, y (batch, L, D); weight (D, width); bias (D)."""
    name: str
    batch: int
    seqlen: int
    dim: int
    width: int
    io: str
    has_bias: bool = True
    silu: bool = True
    x: Dist = Dist(NORMAL, 0.0, 1.0)
    w: Dist = Dist(NORMAL, 0.0, 0.5)
    b: Dist = Dist(NORMAL, 0.0, 1.0)

    def algorithmic_bytes(self) -> int:
        """x read once, y written once (io dtype); weights and bias once."""
        e = 2 if self.io == "bf16" else 4
        return 2 * e * self.batch * self.seqlen * self.dim + 4 * self.dim * (self.width + (1 if self.has_bias else 0))


@dataclass(frozen=True)
class BlockSpec:
    """A Mamba block: u (batch, L, d_model) -> in_proj (2E) -> conv (width k)
    + SiLU -> x_proj (B, C, dt of rank R) -> dt_proj (E) -> scan with
    softplus(delta + b_dt), D skip and SiLU(z) gate -> out_proj (d_model)."""
    name: str
    batch: int
    seqlen: int
    d_model: int
    d_inner: int
    dstate: int
    dt_rank: int
    d_conv: int
    io: str = "bf16"

    @property
    def xproj_width(self) -> int:
        """B, C, dt columns of x_proj, padded with zero rows to a multiple of 8."""
        w = 2 * self.dstate + self.dt_rank
        return (w + 7) // 8 * 8

    def gemm_flops(self) -> float:
        t = self.batch * self.seqlen
        E, M = self.d_inner, self.d_model
        return 2.0 * t * (M * 2 * E + E * (2 * self.dstate + self.dt_rank) + self.dt_rank * E + E * M)


@dataclass(frozen=True)
class SSDSpec:
    """SSD (scalar A per head) problem: x, y (batch, L, H, P); delta (batch, L, H);
    A (H); B, C (batch, L, G, N); D (H)."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    io: str
    has_D: bool
    A: Dist
    delta: Dist
    euler: bool = False
    x: Dist = Dist(NORMAL, 0.0, 1.0)
    B: Dist = Dist(NORMAL, 0.0, 1.0)
    C: Dist = Dist(NORMAL, 0.0, 1.0)
    Dskip: Dist = Dist(NORMAL, 0.0, 1.0)


# The five workloads: a tiny fp32 scan, a Mamba-130M-shaped layer, a
# Mamba-2.8B-shaped layer, a 1M-token fp32 scan and a Mamba-2 (2.7B-shaped)
# SSD layer.
TINY = ScanSpec("tiny_b1_l64_d4_n4_f32", 1, 64, 4, 4, "f32", False, True,
                A=Dist(NEG_EXP_UNIFORM, -1.0, 1.0), delta=Dist(SOFTPLUS_NORMAL, -2.0, 1.0))
MAMBA130M = ScanSpec("mamba130m_b8_l2048_d1536_n16_bf16", 8, 2048, 1536, 16, "bf16", True, True,
                     A=Dist(NEG_IDX, period=16), delta=Dist(SOFTPLUS_NORMAL, -3.0, 1.0))
MAMBA2_8B = ScanSpec("mamba2.8b_b4_l4096_d5120_n16_bf16", 4, 4096, 5120, 16, "bf16", True, True,
                     A=Dist(NEG_IDX, period=16), delta=Dist(SOFTPLUS_NORMAL, -3.0, 1.0))
LONG1M = ScanSpec("long1m_b1_l1048576_d1536_n16_f32", 1, 1 << 20, 1536, 16, "f32", False, False,
                  A=Dist(NEG_IDX, period=16), delta=Dist(SOFTPLUS_NORMAL, -4.0, 1.0))
SSD2_7B = SSDSpec("ssd2.7b_b4_l4096_h80_p64_n64_g1_q256_bf16", 4, 4096, 80, 64, 64, 1, 256, "bf16", True,
                  A=Dist(NEG_EXP_UNIFORM, 0.0, 2.7), delta=Dist(SOFTPLUS_NORMAL, -3.0, 1.0))

# One decode step of the Mamba-2.8B-shaped layer for 64 concurrent sequences
# (seqlen 1: the state (64, 5120, 16) fp32 is read and written in place).
DECODE2_8B = ScanSpec("decode_mamba2.8b_b64_d5120_n16_bf16", 64, 1, 5120, 16, "bf16", True, True,
                      A=Dist(NEG_IDX, period=16), delta=Dist(SOFTPLUS_NORMAL, -3.0, 1.0))

# One Mamba-2.8B-shaped block (d_model 2560, expand 2, N 16, conv width 4;
# the rank of the step-size projection is 1, as in the block listing).
BLOCK2_8B = BlockSpec("block_mamba2.8b_b4_l4096_dm2560_e5120_n16_r1", 4, 4096, 2560, 5120, 16, 1, 4)

# The Mamba-2.8B layer's Conv1D (width 4) in front of its scan.
CONV2_8B = ConvSpec("conv_mamba2.8b_b4_l4096_d5120_w4_bf16", 4, 4096, 5120, 4, "bf16")

SCAN_CONFIGS = {s.name: s for s in (TINY, MAMBA130M, MAMBA2_8B, LONG1M)}


def scan_spec(base: ScanSpec, **kw) -> ScanSpec:
    """Same distributions as `base`, other sizes/flags."""
    if "name" not in kw:
        kw["name"] = base.name + "_" + "_".join("%s%s" % (k, v) for k, v in sorted(kw.items()))
    return replace(base, **kw)


def ssd_spec(base: SSDSpec, **kw) -> SSDSpec:
    if "name" not in kw:
        kw["name"] = base.name + "_" + "_".join("%s%s" % (k, v) for k, v in sorted(kw.items()))
    return replace(base, **kw)


def scan_inputs(s: ScanSpec, seed: int = 0) -> dict:
    """Host arrays for a scan problem.  Keys: x, delta, A, B, C, D, z (absent if off)."""
    io = s.io
    out = {
        "x": fill((s.batch, s.seqlen, s.dim), s.x, io, seed, STREAM["x"]),
        "delta": fill((s.batch, s.seqlen, s.dim), s.delta, io, seed, STREAM["delta"]),
        "A": fill((s.dim, s.dstate), s.A, "f32", seed, STREAM["A"]),
        "B": fill((s.batch, s.seqlen, s.dstate), s.B, io, seed, STREAM["B"]),
        "C": fill((s.batch, s.seqlen, s.dstate), s.C, io, seed, STREAM["C"]),
    }
    if s.has_D:
        out["D"] = fill((s.dim,), s.Dskip, "f32", seed, STREAM["D"])
    if s.has_z:
        out["z"] = fill((s.batch, s.seqlen, s.dim), s.z, io, seed, STREAM["z"])
    return out


def conv_spec(base: ConvSpec, **kw) -> ConvSpec:
    if "name" not in kw:
        kw["name"] = base.name + "_" + "_".join("%s%s" % (k, v) for k, v in sorted(kw.items()))
    return replace(base, **kw)


def conv_inputs(s: ConvSpec, seed: int = 0) -> dict:
    """Host arrays: x (batch, L, D) io; weight (D, width) fp32; bias (D,) fp32 if on."""
    out = {"x": fill((s.batch, s.seqlen, s.dim), s.x, s.io, seed, STREAM["x"]),
           "weight": fill((s.dim, s.width), s.w, "f32", seed, STREAM["conv_w"])}
    if s.has_bias:
        out["bias"] = fill((s.dim,), s.b, "f32", seed, STREAM["conv_b"])
    return out


def block_spec(base: BlockSpec, **kw) -> BlockSpec:
    if "name" not in kw:
        kw["name"] = base.name + "_" + "_".join("%s%s" % (k, v) for k, v in sorted(kw.items()))
    return replace(base, **kw)


def block_inputs(s: BlockSpec, seed: int = 0) -> dict:
    """Input u and random-init weights of the block (projection weights in the
    io dtype, (out, in) layout; the rest fp32):
      W_in (2E, M) ~ N(0, 1/M); conv_w (E, k) ~ N(0, 1/4), conv_b ~ N(0, 1);
      W_x (xproj_width, E) ~ N(0, 1/E), rows B | C | dt, zero padding rows;
      W_dt (E, R) ~ N(0, 1/R); b_dt (E) ~ N(-4, 1) (softplus(-4) ~ 0.018);
      A (E, N) = -(n+1); D (E) ~ N(0, 1); W_out (M, E) ~ N(0, 1/E).
    """
    M, E, N, R, io = s.d_model, s.d_inner, s.dstate, s.dt_rank, s.io
    wx = fill((s.xproj_width, E), Dist(NORMAL, 0.0, E ** -0.5), io, seed, STREAM["w_x"])
    wx[2 * N + R:] = 0
    return {
        "u": fill((s.batch, s.seqlen, M), Dist(NORMAL, 0.0, 1.0), io, seed, STREAM["u"]),
        "W_in": fill((2 * E, M), Dist(NORMAL, 0.0, M ** -0.5), io, seed, STREAM["w_in"]),
        "conv_w": fill((E, s.d_conv), Dist(NORMAL, 0.0, 0.5), "f32", seed, STREAM["conv_w"]),
        "conv_b": fill((E,), Dist(NORMAL, 0.0, 1.0), "f32", seed, STREAM["conv_b"]),
        "W_x": wx,
        "W_dt": fill((E, R), Dist(NORMAL, 0.0, R ** -0.5), io, seed, STREAM["w_dt"]),
        "b_dt": fill((E,), Dist(NORMAL, -4.0, 1.0), "f32", seed, STREAM["delta_bias"]),
        "A": fill((E, N), Dist(NEG_IDX, period=N), "f32", seed, STREAM["A"]),
        "D": fill((E,), Dist(NORMAL, 0.0, 1.0), "f32", seed, STREAM["D"]),
        "W_out": fill((M, E), Dist(NORMAL, 0.0, E ** -0.5), io, seed, STREAM["w_out"]),
    }


def delta_bias_input(dim: int, seed: int = 0, dist: Dist = Dist(NORMAL, -4.0, 1.0)) -> np.ndarray:
    """A per-channel fp32 bias for the softplus step-size transform."""
    return fill((dim,), dist, "f32", seed, STREAM["delta_bias"])


def ssd_inputs(s: SSDSpec, seed: int = 0) -> dict:
    io = s.io
    out = {
        "x": fill((s.batch, s.seqlen, s.nheads, s.headdim), s.x, io, seed, STREAM["x"]),
        "delta": fill((s.batch, s.seqlen, s.nheads), s.delta, io, seed, STREAM["delta"]),
        "A": fill((s.nheads,), s.A, "f32", seed, STREAM["A"]),
        "B": fill((s.batch, s.seqlen, s.ngroups, s.dstate), s.B, io, seed, STREAM["B"]),
        "C": fill((s.batch, s.seqlen, s.ngroups, s.dstate), s.C, io, seed, STREAM["C"]),
    }
    if s.has_D:
        out["D"] = fill((s.nheads,), s.Dskip, "f32", seed, STREAM["D"])
    return out


def state_input(shape, seed: int = 0) -> np.ndarray:
    """An fp32 initial state h0, N(0,1)."""
    return fill(shape, Dist(NORMAL, 0.0, 1.0), "f32", seed, STREAM["h0"])
