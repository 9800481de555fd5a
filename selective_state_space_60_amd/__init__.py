"""Python binding of libssm (include/ssm.h): the selective scan (S6) and the
Mamba-2 SSD chunked form on MI355X.

Argument marshalling only: every step of the computation runs in the gfx950
kernels of ``libssm.so``.  PyTorch supplies device memory and the current HIP
stream.  There is no CPU fallback: if the library is missing this module
raises on import.  Build it with ``python -m selective_state_space_60_amd.build``
or ``__graft_entry__.build()``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm.so")

SSM_OK, SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_DTYPE, SSM_ERR_STRIDE, SSM_ERR_ALIGN, SSM_ERR_ALIAS, \
    SSM_ERR_UNSUPPORTED, SSM_ERR_WORKSPACE, SSM_ERR_HIP = range(10)
SSM_F32, SSM_BF16, SSM_F16 = 0, 1, 2
SSM_HAS_Z, SSM_HAS_D, SSM_DISC_EULER, SSM_HAS_H0, SSM_WANT_HLAST = 1, 2, 4, 8, 16
SSM_DELTA_SOFTPLUS, SSM_HAS_DELTA_BIAS, SSM_HAS_BIAS, SSM_SILU = 32, 64, 128, 256
SSM_WANT_CKPT, SSM_HAS_CKPT, SSM_HAS_SSD_FWD = 512, 1024, 2048
ABI_VERSION = 5
MAX_DIMS = 5

# Every function include/ssm.h declares.
EXPORTS = ("ssm_abi_version", "ssm_status_string", "ssm_last_hip_error", "ssm_selective_scan_workspace_size",
           "ssm_selective_scan_fwd", "ssm_ssd_chunk_workspace_size", "ssm_ssd_chunk_fwd", "ssm_ssd_chunk_cumsum",
           "ssm_ssd_chunk_state", "ssm_ssd_state_passing", "ssm_ssd_chunk_scan", "ssm_selective_state_update",
           "ssm_causal_conv1d_fwd", "ssm_selective_scan_bwd_workspace_size", "ssm_selective_scan_bwd",
           "ssm_ssd_bwd_workspace_size", "ssm_ssd_bwd", "ssm_selective_scan_fwd_noalloc")


class TensorDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * MAX_DIMS),
                ("stride", ctypes.c_int64 * MAX_DIMS)]


_SCAN_T = ("x", "delta", "A", "B", "C", "D", "z", "y", "h0", "h_last", "delta_bias", "ckpt")
_SSD_T = ("x", "delta", "A", "B", "C", "D", "y", "h0", "h_last")
_UPD_T = ("x", "delta", "A", "B", "C", "D", "z", "y", "state", "delta_bias")
_CONV_T = ("x", "weight", "bias", "y")
_BWD_IN = ("x", "delta", "A", "B", "C", "D", "z", "h0", "delta_bias", "dy")
_BWD_OUT = ("dx", "ddelta", "dz", "dA", "dB", "dC", "dD", "dh0", "ddelta_bias")
_SSD_BWD_IN = ("x", "delta", "A", "B", "C", "D", "h0", "dy")
_SSD_BWD_OUT = ("dx", "ddelta", "dA", "dB", "dC", "dD", "dh0")
_SSD_FWD_SAVED = ("A_cum", "beta", "states")   # the forward's intermediates the backward can take


class ScanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("flags", ctypes.c_uint32)] + [(n, TensorDesc) for n in _SCAN_T]


class ScanPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _SCAN_T]


class SSDDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("flags", ctypes.c_uint32)] + [(n, TensorDesc) for n in _SSD_T]


class SSDPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _SSD_T]


class UpdateDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("flags", ctypes.c_uint32)] + [(n, TensorDesc) for n in _UPD_T]


class UpdatePtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _UPD_T]


class ConvDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("width", ctypes.c_int64), ("flags", ctypes.c_uint32)] + [(n, TensorDesc) for n in _CONV_T]


class ConvPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _CONV_T]


class ScanBwdDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("flags", ctypes.c_uint32)] + [(n, TensorDesc) for n in
                                                                           _BWD_IN + _BWD_OUT + ("ckpt",)]


class ScanBwdPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _BWD_IN + _BWD_OUT + ("ckpt",)]


class SSDBwdDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("flags", ctypes.c_uint32)] + [(n, TensorDesc) for n in
                                                                         _SSD_BWD_IN + _SSD_BWD_OUT]


class SSDBwdPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _SSD_BWD_IN + _SSD_BWD_OUT + _SSD_FWD_SAVED]


class SSMError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().ssm_status_string(status).decode()
        if status == SSM_ERR_HIP:
            msg += " (hipError_t %d)" % lib().ssm_last_hip_error()
        super().__init__("%s: %s" % (where, msg))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libssm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libssm.so is not built (run __graft_entry__.build()): " + LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, vp, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
        L.ssm_abi_version.restype = ctypes.c_int
        L.ssm_status_string.restype = ctypes.c_char_p
        L.ssm_status_string.argtypes = [ctypes.c_int]
        L.ssm_last_hip_error.restype = ctypes.c_int
        L.ssm_selective_scan_workspace_size.argtypes = [P(ScanDesc), P(sz)]
        L.ssm_selective_scan_fwd.argtypes = [P(ScanDesc), P(ScanPtrs), vp, sz, vp]
        L.ssm_selective_scan_fwd_noalloc.argtypes = [P(ScanDesc), P(ScanPtrs), vp]
        L.ssm_ssd_chunk_workspace_size.argtypes = [P(SSDDesc), P(sz)]
        L.ssm_ssd_chunk_fwd.argtypes = [P(SSDDesc), P(SSDPtrs), vp, sz, vp]
        L.ssm_ssd_chunk_cumsum.argtypes = [P(SSDDesc), P(SSDPtrs), vp, vp, vp]
        L.ssm_ssd_chunk_state.argtypes = [P(SSDDesc), P(SSDPtrs), vp, vp, vp, vp]
        L.ssm_ssd_state_passing.argtypes = [P(SSDDesc), P(SSDPtrs), vp, vp, vp, vp]
        L.ssm_ssd_chunk_scan.argtypes = [P(SSDDesc), P(SSDPtrs), vp, vp, vp, vp]
        L.ssm_selective_state_update.argtypes = [P(UpdateDesc), P(UpdatePtrs), vp]
        L.ssm_causal_conv1d_fwd.argtypes = [P(ConvDesc), P(ConvPtrs), vp]
        L.ssm_selective_scan_bwd_workspace_size.argtypes = [P(ScanBwdDesc), P(sz)]
        L.ssm_selective_scan_bwd.argtypes = [P(ScanBwdDesc), P(ScanBwdPtrs), vp, sz, vp]
        L.ssm_ssd_bwd_workspace_size.argtypes = [P(SSDBwdDesc), P(sz)]
        L.ssm_ssd_bwd.argtypes = [P(SSDBwdDesc), P(SSDBwdPtrs), vp, sz, vp]
        for name in EXPORTS[3:]:
            getattr(L, name).restype = ctypes.c_int
        if L.ssm_abi_version() != ABI_VERSION:
            raise ImportError("libssm ABI version mismatch")
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().ssm_abi_version()


def status_string(status: int) -> str:
    return lib().ssm_status_string(status).decode()


def _check(status: int, where: str):
    if status != SSM_OK:
        raise SSMError(status, where)


_DT = {torch.float32: SSM_F32, torch.bfloat16: SSM_BF16, torch.float16: SSM_F16}


def tensor_desc(t) -> TensorDesc:
    d = TensorDesc()
    if t is None:
        return d
    d.dtype = _DT.get(t.dtype, -1)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# -------------------------------------------------------------------- scan

def _delta_flags(delta_softplus, delta_bias):
    if delta_bias is not None and not delta_softplus:
        raise ValueError("delta_bias is only used with delta_softplus=True")
    return (SSM_DELTA_SOFTPLUS if delta_softplus else 0) | (SSM_HAS_DELTA_BIAS if delta_bias is not None else 0)


def scan_desc(x, delta, A, B, C, D=None, z=None, y=None, h0=None, h_last=None, euler=False,
              delta_softplus=False, delta_bias=None, ckpt=None) -> ScanDesc:
    d = ScanDesc()
    d.batch, d.seqlen, d.dim = x.shape
    d.dstate = A.shape[-1]
    d.flags = ((SSM_HAS_Z if z is not None else 0) | (SSM_HAS_D if D is not None else 0) |
               (SSM_DISC_EULER if euler else 0) | (SSM_HAS_H0 if h0 is not None else 0) |
               (SSM_WANT_HLAST if h_last is not None else 0) | _delta_flags(delta_softplus, delta_bias) |
               (SSM_WANT_CKPT if ckpt is not None else 0))
    for name, t in zip(_SCAN_T, (x, delta, A, B, C, D, z, y, h0, h_last, delta_bias, ckpt)):
        setattr(d, name, tensor_desc(t))
    return d


def scan_ptrs(x, delta, A, B, C, D=None, z=None, y=None, h0=None, h_last=None, delta_bias=None,
              ckpt=None) -> ScanPtrs:
    p = ScanPtrs()
    for name, t in zip(_SCAN_T, (x, delta, A, B, C, D, z, y, h0, h_last, delta_bias, ckpt)):
        setattr(p, name, _p(t))
    return p


def scan_ckpt(batch: int, seqlen: int, dim: int, dstate: int, device="cuda"):
    """An uninitialised checkpoint buffer for selective_scan_fwd(ckpt=...) and
    selective_scan_bwd(ckpt=...): the state before every 16-step tile."""
    return torch.empty((batch, (seqlen + 15) // 16, dim, dstate), dtype=torch.float32, device=device)


def selective_scan_workspace_size(desc: ScanDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().ssm_selective_scan_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "ssm_selective_scan_workspace_size")
    return n.value


def selective_scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, euler=False, want_hlast=False,
                       y_dtype=None, y=None, stream=None, delta_softplus=False, delta_bias=None, ckpt=None):
    """y = selective scan of x (see include/ssm.h).  Returns (y, h_last or None).

    x, delta, z: (batch, L, dim); B, C: (batch, L, dstate); A: (dim, dstate)
    fp32; D: (dim,) fp32; h0: (batch, dim, dstate) fp32.  x/delta/z/B/C are all
    fp32 or all bf16; y defaults to x's dtype.  delta_softplus: the step size
    is softplus(delta + delta_bias) (delta_bias (dim,) fp32, optional).
    ckpt: optional scan_ckpt(...) buffer, filled with the state before every
    16-step tile for selective_scan_bwd(ckpt=...)."""
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    h_last = torch.empty((x.shape[0], x.shape[2], A.shape[-1]), dtype=torch.float32,
                         device=x.device) if want_hlast else None
    desc = scan_desc(x, delta, A, B, C, D, z, y, h0, h_last, euler, delta_softplus, delta_bias, ckpt)
    ptrs = scan_ptrs(x, delta, A, B, C, D, z, y, h0, h_last, delta_bias, ckpt)
    nbytes = selective_scan_workspace_size(desc)
    ws = _workspace(nbytes, x.device)
    _check(lib().ssm_selective_scan_fwd(ctypes.byref(desc), ctypes.byref(ptrs), _p(ws), nbytes, _stream(stream)),
           "ssm_selective_scan_fwd")
    return y, h_last


SCAN_STATIC_SCRATCH_BYTES = 4 << 20  # SSM_SCAN_STATIC_SCRATCH_BYTES


def selective_scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, h0=None, euler=False, want_hlast=False,
                               y_dtype=None, y=None, stream=None, delta_softplus=False, delta_bias=None, ckpt=None):
    """selective_scan_fwd through ssm_selective_scan_fwd_noalloc: no workspace
    is allocated; the library's static device scratch serves as one (calls on
    one GPU must not overlap).  Pass y (and h_last through want_hlast=False)
    preallocated to keep the call free of allocations."""
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    h_last = torch.empty((x.shape[0], x.shape[2], A.shape[-1]), dtype=torch.float32,
                         device=x.device) if want_hlast else None
    desc = scan_desc(x, delta, A, B, C, D, z, y, h0, h_last, euler, delta_softplus, delta_bias, ckpt)
    ptrs = scan_ptrs(x, delta, A, B, C, D, z, y, h0, h_last, delta_bias, ckpt)
    _check(lib().ssm_selective_scan_fwd_noalloc(ctypes.byref(desc), ctypes.byref(ptrs), _stream(stream)),
           "ssm_selective_scan_fwd_noalloc")
    return y, h_last


# --------------------------------------------------------------------- SSD

def ssd_desc(x, delta, A, B, C, chunk, D=None, y=None, h0=None, h_last=None, euler=False) -> SSDDesc:
    d = SSDDesc()
    d.batch, d.seqlen, d.nheads, d.headdim = x.shape
    d.ngroups, d.dstate = B.shape[2], B.shape[3]
    d.chunk = chunk
    d.flags = ((SSM_HAS_D if D is not None else 0) | (SSM_DISC_EULER if euler else 0) |
               (SSM_HAS_H0 if h0 is not None else 0) | (SSM_WANT_HLAST if h_last is not None else 0))
    for name, t in zip(_SSD_T, (x, delta, A, B, C, D, y, h0, h_last)):
        setattr(d, name, tensor_desc(t))
    if y is None:  # steps that do not write y still need a valid descriptor shape
        d.y = tensor_desc(x)
    return d


def ssd_ptrs(x, delta, A, B, C, D=None, y=None, h0=None, h_last=None) -> SSDPtrs:
    p = SSDPtrs()
    for name, t in zip(_SSD_T, (x, delta, A, B, C, D, y, h0, h_last)):
        setattr(p, name, _p(t))
    return p


def ssd_chunk_workspace_size(desc: SSDDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().ssm_ssd_chunk_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "ssm_ssd_chunk_workspace_size")
    return n.value


def ssd_chunk_fwd(x, delta, A, B, C, chunk, D=None, h0=None, euler=False, want_hlast=False, y_dtype=None,
                  y=None, stream=None):
    """SSD forward (see include/ssm.h).  x: (batch, L, H, P) bf16; delta
    (batch, L, H) bf16; A (H,) fp32; B, C (batch, L, G, N) bf16; D (H,) fp32;
    h0 (batch, H, P, N) fp32.  Returns (y, h_last or None)."""
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    h_last = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]), dtype=torch.float32,
                         device=x.device) if want_hlast else None
    desc = ssd_desc(x, delta, A, B, C, chunk, D, y, h0, h_last, euler)
    ptrs = ssd_ptrs(x, delta, A, B, C, D, y, h0, h_last)
    nbytes = ssd_chunk_workspace_size(desc)
    ws = _workspace(nbytes, x.device)
    _check(lib().ssm_ssd_chunk_fwd(ctypes.byref(desc), ctypes.byref(ptrs), _p(ws), nbytes, _stream(stream)),
           "ssm_ssd_chunk_fwd")
    return y, h_last


def _ssd_shapes(x, B, chunk):
    batch, L, H, P = x.shape
    N = B.shape[3]
    nc = (L + chunk - 1) // chunk
    return batch, H, P, N, nc, nc * chunk


def ssd_chunk_cumsum(x, delta, A, B, C, chunk, euler=False, stream=None):
    """Step 1: (A_cum, beta), each (batch, H, nchunks*chunk) fp32."""
    batch, H, P, N, nc, Lp = _ssd_shapes(x, B, chunk)
    A_cum = torch.empty((batch, H, Lp), dtype=torch.float32, device=x.device)
    beta = torch.empty_like(A_cum)
    desc = ssd_desc(x, delta, A, B, C, chunk, euler=euler)
    _check(lib().ssm_ssd_chunk_cumsum(ctypes.byref(desc), ctypes.byref(ssd_ptrs(x, delta, A, B, C)), _p(A_cum),
                                      _p(beta), _stream(stream)), "ssm_ssd_chunk_cumsum")
    return A_cum, beta


def ssd_chunk_state(x, delta, A, B, C, chunk, A_cum, beta, euler=False, stream=None):
    """Step 2: chunk-local states (batch, nchunks, H, P, N) fp32."""
    batch, H, P, N, nc, Lp = _ssd_shapes(x, B, chunk)
    states = torch.empty((batch, nc, H, P, N), dtype=torch.float32, device=x.device)
    desc = ssd_desc(x, delta, A, B, C, chunk, euler=euler)
    _check(lib().ssm_ssd_chunk_state(ctypes.byref(desc), ctypes.byref(ssd_ptrs(x, delta, A, B, C)), _p(A_cum),
                                     _p(beta), _p(states), _stream(stream)), "ssm_ssd_chunk_state")
    return states


def ssd_state_passing(x, delta, A, B, C, chunk, A_cum, states, h0=None, want_hlast=False, euler=False,
                      stream=None):
    """Step 3: (S_in (batch, nchunks, H, P, N) bf16, h_last or None)."""
    batch, H, P, N, nc, Lp = _ssd_shapes(x, B, chunk)
    S_in = torch.empty((batch, nc, H, P, N), dtype=torch.bfloat16, device=x.device)
    h_last = torch.empty((batch, H, P, N), dtype=torch.float32, device=x.device) if want_hlast else None
    desc = ssd_desc(x, delta, A, B, C, chunk, h0=h0, h_last=h_last, euler=euler)
    ptrs = ssd_ptrs(x, delta, A, B, C, h0=h0, h_last=h_last)
    _check(lib().ssm_ssd_state_passing(ctypes.byref(desc), ctypes.byref(ptrs), _p(A_cum), _p(states), _p(S_in),
                                       _stream(stream)), "ssm_ssd_state_passing")
    return S_in, h_last


def ssd_chunk_scan(x, delta, A, B, C, chunk, A_cum, beta, S_in, D=None, euler=False, y_dtype=None, y=None,
                   stream=None):
    """Step 4: y (batch, L, H, P)."""
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    desc = ssd_desc(x, delta, A, B, C, chunk, D=D, y=y, euler=euler)
    ptrs = ssd_ptrs(x, delta, A, B, C, D=D, y=y)
    _check(lib().ssm_ssd_chunk_scan(ctypes.byref(desc), ctypes.byref(ptrs), _p(A_cum), _p(beta), _p(S_in),
                                    _stream(stream)), "ssm_ssd_chunk_scan")
    return y


def ssd_chunk_fwd_train(x, delta, A, B, C, chunk, D=None, h0=None, euler=False, want_hlast=False, y_dtype=None,
                        stream=None):
    """SSD forward by its four steps, keeping what ssd_bwd(..., fwd=saved)
    takes instead of recomputing it.  Returns (y, h_last or None, saved) with
    saved = {"A_cum", "beta", "states", "chunk", "euler"} (the last two let
    ssd_bwd refuse a backward of another chunk size or discretisation)."""
    A_cum, beta = ssd_chunk_cumsum(x, delta, A, B, C, chunk, euler=euler, stream=stream)
    states = ssd_chunk_state(x, delta, A, B, C, chunk, A_cum, beta, euler=euler, stream=stream)
    S_in, h_last = ssd_state_passing(x, delta, A, B, C, chunk, A_cum, states, h0=h0, want_hlast=want_hlast,
                                     euler=euler, stream=stream)
    y = ssd_chunk_scan(x, delta, A, B, C, chunk, A_cum, beta, S_in, D=D, euler=euler, y_dtype=y_dtype,
                       stream=stream)
    return y, h_last, {"A_cum": A_cum, "beta": beta, "states": states, "chunk": chunk, "euler": bool(euler)}


# ------------------------------------------------------------------ decode

def update_desc(x, delta, A, B, C, state, D=None, z=None, y=None, euler=False, delta_softplus=False,
                delta_bias=None) -> UpdateDesc:
    d = UpdateDesc()
    d.batch, d.dim = x.shape
    d.dstate = A.shape[-1]
    d.flags = ((SSM_HAS_Z if z is not None else 0) | (SSM_HAS_D if D is not None else 0) |
               (SSM_DISC_EULER if euler else 0) | _delta_flags(delta_softplus, delta_bias))
    for name, t in zip(_UPD_T, (x, delta, A, B, C, D, z, y, state, delta_bias)):
        setattr(d, name, tensor_desc(t))
    return d


def update_ptrs(x, delta, A, B, C, state, D=None, z=None, y=None, delta_bias=None) -> UpdatePtrs:
    p = UpdatePtrs()
    for name, t in zip(_UPD_T, (x, delta, A, B, C, D, z, y, state, delta_bias)):
        setattr(p, name, _p(t))
    return p


def selective_state_update(state, x, delta, A, B, C, D=None, z=None, euler=False, y_dtype=None, y=None,
                           stream=None, delta_softplus=False, delta_bias=None):
    """One decode step (see include/ssm.h): advances ``state`` (batch, dim,
    dstate) fp32 in place and returns y (batch, dim).  x, delta, z: (batch,
    dim); B, C: (batch, dstate); A: (dim, dstate) fp32; D: (dim,) fp32;
    delta_softplus / delta_bias as in selective_scan_fwd."""
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    desc = update_desc(x, delta, A, B, C, state, D, z, y, euler, delta_softplus, delta_bias)
    ptrs = update_ptrs(x, delta, A, B, C, state, D, z, y, delta_bias)
    _check(lib().ssm_selective_state_update(ctypes.byref(desc), ctypes.byref(ptrs), _stream(stream)),
           "ssm_selective_state_update")
    return y


# -------------------------------------------------------------------- conv

def conv_desc(x, weight, bias=None, y=None, silu=True) -> ConvDesc:
    d = ConvDesc()
    d.batch, d.seqlen, d.dim = x.shape
    d.width = weight.shape[-1]
    d.flags = (SSM_HAS_BIAS if bias is not None else 0) | (SSM_SILU if silu else 0)
    for name, t in zip(_CONV_T, (x, weight, bias, y)):
        setattr(d, name, tensor_desc(t))
    return d


def conv_ptrs(x, weight, bias=None, y=None) -> ConvPtrs:
    p = ConvPtrs()
    for name, t in zip(_CONV_T, (x, weight, bias, y)):
        setattr(p, name, _p(t))
    return p


def causal_conv1d(x, weight, bias=None, silu=True, y_dtype=None, y=None, stream=None):
    """Causal depthwise convolution (+ bias, + SiLU) (see include/ssm.h).
    x: (batch, L, dim) fp32 or bf16; weight: (dim, width) fp32, width <= 8;
    bias: (dim,) fp32.  Returns y (batch, L, dim), x's dtype by default."""
    if y is None:
        y = torch.empty(x.shape, dtype=y_dtype or x.dtype, device=x.device)
    desc = conv_desc(x, weight, bias, y, silu)
    ptrs = conv_ptrs(x, weight, bias, y)
    _check(lib().ssm_causal_conv1d_fwd(ctypes.byref(desc), ctypes.byref(ptrs), _stream(stream)),
           "ssm_causal_conv1d_fwd")
    return y


# ---------------------------------------------------------- scan backward

def selective_scan_bwd(dy, x, delta, A, B, C, D=None, z=None, h0=None, euler=False, delta_softplus=False,
                       delta_bias=None, grad_dtype=None, stream=None, ckpt=None) -> dict:
    """Gradients of sum(dy * y) for y = selective_scan_fwd(x, delta, A, B, C,
    D, z, h0, euler, delta_softplus, delta_bias) (see include/ssm.h).
    ckpt: the forward's checkpoints of the same inputs (selective_scan_fwd(...,
    ckpt=...)); without them the backward recomputes them.

    Returns a dict: dx, ddelta (grad_dtype, default x's dtype), dz (if z), dA
    (dim, dstate), dB, dC (batch, L, dstate), dD (if D), dh0 (if h0),
    ddelta_bias (if delta_bias); the last six fp32."""
    gdt = grad_dtype or x.dtype
    batch, L, dim = x.shape
    N = A.shape[-1]
    dev = x.device
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
    out = {"dx": torch.empty(x.shape, dtype=gdt, device=dev), "ddelta": torch.empty(x.shape, dtype=gdt, device=dev),
           "dz": torch.empty(x.shape, dtype=gdt, device=dev) if z is not None else None,
           "dA": f32(dim, N), "dB": f32(batch, L, N), "dC": f32(batch, L, N),
           "dD": f32(dim) if D is not None else None, "dh0": f32(batch, dim, N) if h0 is not None else None,
           "ddelta_bias": f32(dim) if delta_bias is not None else None}
    ins = (x, delta, A, B, C, D, z, h0, delta_bias, dy)
    d = ScanBwdDesc()
    d.batch, d.seqlen, d.dim, d.dstate = batch, L, dim, N
    d.flags = ((SSM_HAS_Z if z is not None else 0) | (SSM_HAS_D if D is not None else 0) |
               (SSM_DISC_EULER if euler else 0) | (SSM_HAS_H0 if h0 is not None else 0) |
               _delta_flags(delta_softplus, delta_bias) | (SSM_HAS_CKPT if ckpt is not None else 0))
    p = ScanBwdPtrs()
    for name, t in list(zip(_BWD_IN, ins)) + [(k, out[k]) for k in _BWD_OUT] + [("ckpt", ckpt)]:
        setattr(d, name, tensor_desc(t))
        setattr(p, name, _p(t))
    n = ctypes.c_size_t()
    _check(lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)),
           "ssm_selective_scan_bwd_workspace_size")
    ws = _workspace(n.value, dev)
    _check(lib().ssm_selective_scan_bwd(ctypes.byref(d), ctypes.byref(p), _p(ws), n.value, _stream(stream)),
           "ssm_selective_scan_bwd")
    return {k: v for k, v in out.items() if v is not None}


# ----------------------------------------------------------- SSD backward

def ssd_bwd_desc(dy, x, delta, A, B, C, chunk, out: dict, D=None, h0=None, euler=False,
                 has_fwd=False) -> SSDBwdDesc:
    d = SSDBwdDesc()
    d.batch, d.seqlen, d.nheads, d.headdim = x.shape
    d.ngroups, d.dstate = B.shape[2], B.shape[3]
    d.chunk = chunk
    d.flags = (SSM_HAS_D if D is not None else 0) | (SSM_DISC_EULER if euler else 0) | \
        (SSM_HAS_H0 if h0 is not None else 0) | (SSM_HAS_SSD_FWD if has_fwd else 0)
    for name, t in list(zip(_SSD_BWD_IN, (x, delta, A, B, C, D, h0, dy))) + [(k, out.get(k)) for k in _SSD_BWD_OUT]:
        setattr(d, name, tensor_desc(t))
    return d


def ssd_bwd(dy, x, delta, A, B, C, chunk, D=None, h0=None, euler=False, dx_dtype=None, fwd=None,
            stream=None) -> dict:
    """Gradients of sum(dy * y) for y = ssd_chunk_fwd(x, delta, A, B, C,
    chunk, D, h0, euler) (see include/ssm.h).  dy (batch, L, H, P) bf16.
    fwd: the `saved` dict of ssd_chunk_fwd_train on the same inputs, whose
    A_cum, beta and chunk states are then read instead of recomputed.

    Returns a dict: dx (dx_dtype, default x's dtype), ddelta (batch, L, H),
    dA (H,), dB, dC (batch, L, G, N), dD (if D), dh0 (if h0); all but dx fp32."""
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
    out = {"dx": torch.empty(x.shape, dtype=dx_dtype or x.dtype, device=dev), "ddelta": f32(batch, L, H),
           "dA": f32(H), "dB": f32(batch, L, G, N), "dC": f32(batch, L, G, N),
           "dD": f32(H) if D is not None else None, "dh0": f32(batch, H, P, N) if h0 is not None else None}
    d = ssd_bwd_desc(dy, x, delta, A, B, C, chunk, out, D, h0, euler, has_fwd=fwd is not None)
    p = SSDBwdPtrs()
    for name, t in list(zip(_SSD_BWD_IN, (x, delta, A, B, C, D, h0, dy))) + [(k, out[k]) for k in _SSD_BWD_OUT]:
        setattr(p, name, _p(t))
    if fwd is not None:
        # intermediates of another chunk size or discretisation would give wrong gradients
        for k, v in (("chunk", chunk), ("euler", bool(euler))):
            if k in fwd and fwd[k] != v:
                raise ValueError(f"ssd_bwd: fwd was computed with {k}={fwd[k]!r}, this backward has {k}={v!r}")
        # the library sees bare pointers here, so the shapes are checked on this side
        _, _, _, _, nc, Lp = _ssd_shapes(x, B, chunk)
        want = {"A_cum": (batch, H, Lp), "beta": (batch, H, Lp), "states": (batch, nc, H, P, N)}
        for k in _SSD_FWD_SAVED:
            t = fwd[k]
            if tuple(t.shape) != want[k] or t.dtype != torch.float32 or not t.is_contiguous() or t.device != dev:
                raise ValueError(f"ssd_bwd: fwd[{k!r}] must be a contiguous fp32 {want[k]} tensor on {dev}")
            setattr(p, k, _p(t))
    n = ctypes.c_size_t()
    _check(lib().ssm_ssd_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)), "ssm_ssd_bwd_workspace_size")
    ws = _workspace(n.value, dev)
    _check(lib().ssm_ssd_bwd(ctypes.byref(d), ctypes.byref(p), _p(ws), n.value, _stream(stream)), "ssm_ssd_bwd")
    return {k: v for k, v in out.items() if v is not None}
