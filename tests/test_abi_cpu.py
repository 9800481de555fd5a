"""The C ABI without a GPU: libssm.so loads, exports every function that
include/ssm.h declares, and rejects malformed calls on the host before any
HIP call (no compute runs here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ssm = pytest.importorskip("selective_state_space_60_amd")

_torch = pytest.importorskip("torch")
if _torch.cuda.is_available():  # pragma: no cover
    # every call below passes fake device addresses and must be rejected on
    # the host; with a GPU visible a validation gap would launch on them
    pytest.skip("host-validation tests run without a GPU", allow_module_level=True)

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _header_functions():
    text = open(os.path.join(ROOT, "include", "ssm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    lib = ssm.lib()
    declared = _header_functions()
    assert declared == sorted(ssm.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.ssm_abi_version() == ssm.ABI_VERSION == 5


def test_status_strings():
    for s in range(10):
        assert ssm.status_string(s).startswith("SSM_")
    assert ssm.lib().ssm_last_hip_error() == 0


class T:
    """Shape/stride/dtype stand-in for a tensor (no memory)."""

    def __init__(self, shape, dtype="f32", strides=None, ptr=FAKE):
        self.shape = tuple(shape)
        self.dt = {"f32": 0, "bf16": 1, "f16": 2}[dtype]
        if strides is None:
            strides, acc = [], 1
            for s in reversed(shape):
                strides.insert(0, acc)
                acc *= s
        self.strides = tuple(strides)
        self.ptr = ptr


def _td(t):
    d = ssm.TensorDesc()
    if t is None:
        return d
    d.dtype, d.ndim = t.dt, len(t.shape)
    for i, (s, st) in enumerate(zip(t.shape, t.strides)):
        d.shape[i], d.stride[i] = s, st
    return d


def _scan(batch=2, L=16, D=8, N=4, io="bf16", flags=0, **over):
    ts = {"x": T((batch, L, D), io, ptr=1 << 36), "delta": T((batch, L, D), io, ptr=2 << 36),
          "A": T((D, N), ptr=3 << 36), "B": T((batch, L, N), io, ptr=4 << 36),
          "C": T((batch, L, N), io, ptr=5 << 36), "D": T((D,), ptr=6 << 36),
          "z": T((batch, L, D), io, ptr=7 << 36), "y": T((batch, L, D), io, ptr=8 << 36),
          "h0": T((batch, D, N), ptr=9 << 36), "h_last": T((batch, D, N), ptr=10 << 36),
          "delta_bias": T((D,), ptr=11 << 36)}
    ts.update(over)
    d = ssm.ScanDesc()
    d.batch, d.seqlen, d.dim, d.dstate, d.flags = batch, L, D, N, flags
    p = ssm.ScanPtrs()
    for k, t in ts.items():
        setattr(d, k, _td(t))
        setattr(p, k, None if t is None or t.ptr is None else t.ptr)
    return d, p


def _fwd(d, p, ws=None, nbytes=0):
    return ssm.lib().ssm_selective_scan_fwd(ctypes.byref(d), ctypes.byref(p), ws, nbytes, None)


ALL = ssm.SSM_HAS_Z | ssm.SSM_HAS_D | ssm.SSM_HAS_H0 | ssm.SSM_WANT_HLAST


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(p, "x", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "z", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "h_last", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(d, "seqlen", 0), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(d, "dim", -3), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(d, "dstate", 65), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "flags", d.flags | (1 << 20)), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.x, "dtype", 2), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.delta, "dtype", 0), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(d.A, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(d.h0, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.B.shape.__setitem__(2, 5), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(d.C, "ndim", 2), ssm.SSM_ERR_SHAPE),
    (lambda d, p: d.x.stride.__setitem__(2, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: d.delta.stride.__setitem__(0, -1), ssm.SSM_ERR_STRIDE),
    (lambda d, p: d.h_last.stride.__setitem__(1, 8), ssm.SSM_ERR_STRIDE),
    (lambda d, p: d.y.stride.__setitem__(1, 0), ssm.SSM_ERR_STRIDE),
    (lambda d, p: setattr(p, "x", (1 << 36) + 1), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "h0", (9 << 36) + 2), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "y", p.x), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "h_last", p.y + 16), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "y", p.z + 2), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(d, "flags", d.flags & ~ssm.SSM_DELTA_SOFTPLUS), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(p, "delta_bias", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(d.delta_bias, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.delta_bias.shape.__setitem__(0, 9), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(p, "delta_bias", (11 << 36) + 2), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "h_last", p.delta_bias), ssm.SSM_ERR_ALIAS),
])
def test_scan_validation(mutate, status):
    d, p = _scan(flags=ALL | ssm.SSM_DELTA_SOFTPLUS | ssm.SSM_HAS_DELTA_BIAS)
    mutate(d, p)
    assert _fwd(d, p) == status


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(p, "ckpt", None), ssm.SSM_ERR_NULL),
    (lambda d, p: d.ckpt.shape.__setitem__(1, 2), ssm.SSM_ERR_SHAPE),   # ceil(16 / 16) = 1 tile
    (lambda d, p: setattr(d.ckpt, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.ckpt.stride.__setitem__(2, 8), ssm.SSM_ERR_STRIDE),
    (lambda d, p: setattr(p, "ckpt", (12 << 36) + 2), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "ckpt", p.y), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "ckpt", p.h0), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "ckpt", p.h_last), ssm.SSM_ERR_ALIAS),
])
def test_scan_ckpt_validation(mutate, status):
    d, p = _scan(flags=ALL | ssm.SSM_WANT_CKPT, ckpt=T((2, 1, 8, 4), ptr=12 << 36))
    mutate(d, p)
    assert _fwd(d, p) == status


def _scan_bwd(batch=2, L=40, D=8, N=4, io="bf16", flags=0, **over):
    nt = (L + 15) // 16
    ts = {"x": T((batch, L, D), io, ptr=1 << 36), "delta": T((batch, L, D), io, ptr=2 << 36),
          "A": T((D, N), ptr=3 << 36), "B": T((batch, L, N), io, ptr=4 << 36),
          "C": T((batch, L, N), io, ptr=5 << 36), "D": T((D,), ptr=6 << 36),
          "z": T((batch, L, D), io, ptr=7 << 36), "h0": T((batch, D, N), ptr=8 << 36),
          "delta_bias": T((D,), ptr=9 << 36), "dy": T((batch, L, D), io, ptr=10 << 36),
          "dx": T((batch, L, D), io, ptr=11 << 36), "ddelta": T((batch, L, D), io, ptr=12 << 36),
          "dz": T((batch, L, D), io, ptr=13 << 36), "dA": T((D, N), ptr=14 << 36),
          "dB": T((batch, L, N), ptr=15 << 36), "dC": T((batch, L, N), ptr=16 << 36),
          "dD": T((D,), ptr=17 << 36), "dh0": T((batch, D, N), ptr=18 << 36),
          "ddelta_bias": T((D,), ptr=19 << 36), "ckpt": T((batch, nt, D, N), ptr=20 << 36)}
    ts.update(over)
    d = ssm.ScanBwdDesc()
    d.batch, d.seqlen, d.dim, d.dstate, d.flags = batch, L, D, N, flags
    p = ssm.ScanBwdPtrs()
    for k, t in ts.items():
        setattr(d, k, _td(t))
        setattr(p, k, None if t is None or t.ptr is None else t.ptr)
    return d, p


BWD_ALL = (ssm.SSM_HAS_Z | ssm.SSM_HAS_D | ssm.SSM_HAS_H0 | ssm.SSM_DELTA_SOFTPLUS | ssm.SSM_HAS_DELTA_BIAS |
           ssm.SSM_HAS_CKPT)


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_WANT_HLAST), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_WANT_CKPT), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "dstate", 65), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(p, "dy", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "dz", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "ckpt", None), ssm.SSM_ERR_NULL),
    (lambda d, p: d.ckpt.shape.__setitem__(1, 2), ssm.SSM_ERR_SHAPE),   # ceil(40 / 16) = 3 tiles
    (lambda d, p: setattr(d.ckpt, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(d.dA, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.dB.stride.__setitem__(2, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: setattr(p, "ckpt", (20 << 36) + 2), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "dx", p.ckpt), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "dB", p.dC), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "ddelta", p.delta), ssm.SSM_ERR_ALIAS),
])
def test_scan_bwd_validation(mutate, status):
    d, p = _scan_bwd(flags=BWD_ALL)
    mutate(d, p)
    assert ssm.lib().ssm_selective_scan_bwd(ctypes.byref(d), ctypes.byref(p), 30 << 36, 1 << 40, None) == status


def test_scan_bwd_workspace_without_checkpoints():
    # given the forward's checkpoints, the backward keeps none of its own
    n = ctypes.c_size_t()
    d, _ = _scan_bwd(batch=4, L=4096, D=5120, N=16, flags=ssm.SSM_HAS_Z | ssm.SSM_HAS_D)
    assert ssm.lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == ssm.SSM_OK
    with_ck = n.value
    d, _ = _scan_bwd(batch=4, L=4096, D=5120, N=16, flags=ssm.SSM_HAS_Z | ssm.SSM_HAS_D | ssm.SSM_HAS_CKPT)
    assert ssm.lib().ssm_selective_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == ssm.SSM_OK
    assert with_ck - n.value == 4 * 256 * 5120 * 16 * 4


def test_scan_null_descriptor():
    assert ssm.lib().ssm_selective_scan_fwd(None, None, None, 0, None) == ssm.SSM_ERR_NULL
    n = ctypes.c_size_t()
    assert ssm.lib().ssm_selective_scan_workspace_size(None, ctypes.byref(n)) == ssm.SSM_ERR_NULL


def test_scan_workspace_plan():
    """Wide problems need no workspace; long narrow ones split the sequence."""
    d, p = _scan(batch=4, L=4096, D=5120, N=16)
    assert ssm.selective_scan_workspace_size(d) == 0
    d, p = _scan(batch=1, L=1 << 20, D=1536, N=16, io="f32", flags=0)
    n = ssm.selective_scan_workspace_size(d)
    assert n > 0
    # a missing or short workspace is rejected before any launch
    assert _fwd(d, p, None, 0) == ssm.SSM_ERR_WORKSPACE
    assert _fwd(d, p, 12 << 36, n - 1) == ssm.SSM_ERR_WORKSPACE
    assert _fwd(d, p, (12 << 36) + 16, n) == ssm.SSM_ERR_ALIGN


def test_scan_broadcast_A_accepted_by_validation():
    # stride-0 A is a valid input: validation passes, so the call would launch;
    # check only the workspace query (pure host code)
    d, p = _scan(A=T((8, 4), strides=(0, 1)))
    assert ssm.selective_scan_workspace_size(d) == 0


def _ssd(batch=1, L=100, H=4, P=64, N=64, G=1, Q=64, flags=0, **over):
    ts = {"x": T((batch, L, H, P), "bf16", ptr=1 << 36), "delta": T((batch, L, H), "bf16", ptr=2 << 36),
          "A": T((H,), ptr=3 << 36), "B": T((batch, L, G, N), "bf16", ptr=4 << 36),
          "C": T((batch, L, G, N), "bf16", ptr=5 << 36), "D": T((H,), ptr=6 << 36),
          "y": T((batch, L, H, P), "bf16", ptr=8 << 36), "h0": T((batch, H, P, N), ptr=9 << 36),
          "h_last": T((batch, H, P, N), ptr=10 << 36)}
    ts.update(over)
    d = ssm.SSDDesc()
    d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.ngroups, d.chunk, d.flags = batch, L, H, P, N, G, Q, flags
    p = ssm.SSDPtrs()
    for k, t in ts.items():
        setattr(d, k, _td(t))
        setattr(p, k, None if t is None else t.ptr)
    return d, p


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(d, "chunk", 100), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "headdim", 32), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "dstate", 96), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: (setattr(d, "dstate", 256), setattr(d, "chunk", 256)), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "dstate", 128), ssm.SSM_ERR_SHAPE),  # B, C, h0 still have 64 states
    (lambda d, p: setattr(d, "ngroups", 3), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_HAS_Z), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.x, "dtype", 0), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.B, "dtype", 0), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.C.stride.__setitem__(3, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: setattr(p, "D", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "y", p.x), ssm.SSM_ERR_ALIAS),
])
def test_ssd_validation(mutate, status):
    d, p = _ssd(flags=ssm.SSM_HAS_D | ssm.SSM_HAS_H0 | ssm.SSM_WANT_HLAST)
    mutate(d, p)
    n = 1 << 30
    assert ssm.lib().ssm_ssd_chunk_fwd(ctypes.byref(d), ctypes.byref(p), 12 << 36, n, None) == status


def _ssd_bwd(batch=1, L=100, H=4, P=64, N=64, G=1, Q=64, flags=0, **over):
    ts = {"x": T((batch, L, H, P), "bf16", ptr=1 << 36), "delta": T((batch, L, H), "bf16", ptr=2 << 36),
          "A": T((H,), ptr=3 << 36), "B": T((batch, L, G, N), "bf16", ptr=4 << 36),
          "C": T((batch, L, G, N), "bf16", ptr=5 << 36), "D": T((H,), ptr=6 << 36),
          "h0": T((batch, H, P, N), ptr=7 << 36), "dy": T((batch, L, H, P), "bf16", ptr=8 << 36),
          "dx": T((batch, L, H, P), "bf16", ptr=9 << 36), "ddelta": T((batch, L, H), ptr=10 << 36),
          "dA": T((H,), ptr=11 << 36), "dB": T((batch, L, G, N), ptr=12 << 36),
          "dC": T((batch, L, G, N), ptr=13 << 36), "dD": T((H,), ptr=14 << 36),
          "dh0": T((batch, H, P, N), ptr=15 << 36)}
    ts.update(over)
    d = ssm.SSDBwdDesc()
    d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.ngroups, d.chunk, d.flags = batch, L, H, P, N, G, Q, flags
    p = ssm.SSDBwdPtrs()
    for k, t in ts.items():
        setattr(d, k, _td(t))
        setattr(p, k, None if t is None else t.ptr)
    return d, p


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_WANT_HLAST), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_HAS_Z), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "chunk", 32), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "headdim", 32), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "dstate", 128), ssm.SSM_ERR_SHAPE),   # B, C, h0 still have 64 states
    (lambda d, p: setattr(d.dy, "dtype", 0), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(d.ddelta, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(d.dB, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.dC.stride.__setitem__(3, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: d.dy.stride.__setitem__(3, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: setattr(p, "dD", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "dh0", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "dy", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "dx", p.x), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "dC", p.dB), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "dh0", p.dh0 + 4), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "dx", p.dx + 2), ssm.SSM_ERR_ALIGN),
    # chunk rows of x and dy are addressed with 32-bit byte offsets
    (lambda d, p: (d.x.stride.__setitem__(1, 1 << 24), d.x.stride.__setitem__(0, 1 << 32)), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: (d.dy.stride.__setitem__(1, 1 << 24), d.dy.stride.__setitem__(0, 1 << 32)), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: (d.dy.stride.__setitem__(1, 1 << 20), d.dy.stride.__setitem__(0, 1 << 28)), ssm.SSM_OK),
])
def test_ssd_bwd_validation(mutate, status):
    d, p = _ssd_bwd(flags=ssm.SSM_HAS_D | ssm.SSM_HAS_H0)
    mutate(d, p)
    n = 1 << 40
    if status == ssm.SSM_OK:   # valid: stop before any launch with a too-small workspace
        status, n = ssm.SSM_ERR_WORKSPACE, 256
    assert ssm.lib().ssm_ssd_bwd(ctypes.byref(d), ctypes.byref(p), 16 << 36, n, None) == status


# batch 1, L 100, 4 heads, chunk 64: A_cum, beta (1, 4, 128) fp32; states (1, 2, 4, 64, 64) fp32
_FWD = {"A_cum": 17 << 36, "beta": 18 << 36, "states": 19 << 36}


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(p, "A_cum", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "states", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "beta", p.beta + 4), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "states", p.states + 8), ssm.SSM_ERR_ALIGN),
    # each buffer's extent: A_cum is 1 * 4 * 128 * 4 = 2048 bytes, states 2 * 4 * 4096 * 4 bytes
    (lambda d, p: setattr(p, "dA", p.A_cum + 2032), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "dA", p.A_cum + 2048), ssm.SSM_OK),
    (lambda d, p: setattr(p, "dh0", p.states + 2 * 4 * 4096 * 4 - 16), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "ddelta", p.beta), ssm.SSM_ERR_ALIAS),
])
def test_ssd_bwd_fwd_validation(mutate, status):
    d, p = _ssd_bwd(flags=ssm.SSM_HAS_D | ssm.SSM_HAS_H0 | ssm.SSM_HAS_SSD_FWD)
    for k, v in _FWD.items():
        setattr(p, k, v)
    mutate(d, p)
    if status == ssm.SSM_OK:   # valid: stop before any launch with a too-small workspace
        status = ssm.SSM_ERR_WORKSPACE
        n = 256
    else:
        n = 1 << 40
    assert ssm.lib().ssm_ssd_bwd(ctypes.byref(d), ctypes.byref(p), 16 << 36, n, None) == status


def test_ssd_bwd_dstate_limit():
    # as in the forward: 96 states are not a supported size, 256 states not with chunk 256
    d, p = _ssd_bwd(N=96)
    assert ssm.lib().ssm_ssd_bwd(ctypes.byref(d), ctypes.byref(p), 16 << 36, 1 << 40, None) == \
        ssm.SSM_ERR_UNSUPPORTED
    d, p = _ssd_bwd(N=256, Q=256)
    assert ssm.lib().ssm_ssd_bwd(ctypes.byref(d), ctypes.byref(p), 16 << 36, 1 << 40, None) == \
        ssm.SSM_ERR_UNSUPPORTED


def test_ssd_bwd_workspace():
    d, p = _ssd_bwd(batch=4, L=4096, H=80, Q=256, flags=ssm.SSM_HAS_D)
    n = ctypes.c_size_t()
    assert ssm.lib().ssm_ssd_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == ssm.SSM_OK
    nc, E = 16, 64 * 64
    # chunk 256, 64 states: heads per workgroup that give the fewest rounds of
    # one workgroup per compute unit x (heads + 1): 20, so 4 head blocks and
    # 4 * 16 * 4 = 256 workgroups, one round
    HB = 20
    nhb = 4
    # the chunk-end decay gradient: 8 partial sums per (batch, head, chunk),
    # one per 8-row workgroup of the state pass (up to 32 chunks)
    # (no fp32 copy of the entering states: up to 32 chunks the state pass
    # keeps them in registers)
    want = (2 * 4 * 80 * 4096 * 4 + 2 * 4 * nc * 80 * E * 4 + 3 * 4 * nc * 80 * E * 2 + 4 * 80 * nc * 8 * 4 +
            5 * 4 * 80 * 4096 * 4 + 2 * 4 * nc * 80 * 4 + 2 * nhb * 4 * 4096 * 64 * 4)
    assert HB * nhb == 80
    assert n.value == want
    assert ssm.lib().ssm_ssd_bwd(ctypes.byref(d), ctypes.byref(p), 16 << 36, n.value - 1, None) == \
        ssm.SSM_ERR_WORKSPACE
    # with the forward's A_cum, beta and states given, their space is not taken
    d.flags |= ssm.SSM_HAS_SSD_FWD
    m = ctypes.c_size_t()
    assert ssm.lib().ssm_ssd_bwd_workspace_size(ctypes.byref(d), ctypes.byref(m)) == ssm.SSM_OK
    assert n.value - m.value == 2 * 4 * 80 * 4096 * 4 + 4 * nc * 80 * E * 4


@pytest.mark.parametrize("batch,L,H,Q,nhb", [
    (4, 4096, 80, 256, 4),   # 64 (batch, chunk) pairs: 20 heads per workgroup, 256 workgroups
    (4, 4096, 80, 128, 2),   # 128 pairs: 40 heads, 256 workgroups
    (1, 4096, 80, 256, 16),  # 16 pairs: 5 heads, 256 workgroups
    (1, 300, 8, 64, 8),      # 5 pairs: one head per workgroup (one round either way)
])
def test_ssd_bwd_head_blocks(batch, L, H, Q, nhb):
    # the dB, dC partial sums (two fp32 (nhb, batch, L, G, N) buffers, the last
    # part of the workspace) count the head blocks the planner chose: the head
    # count that minimises (rounds of 256 workgroups) x (heads + 1)
    d, _ = _ssd_bwd(batch=batch, L=L, H=H, Q=Q)
    n = ctypes.c_size_t()
    assert ssm.lib().ssm_ssd_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == ssm.SSM_OK
    part = 4 * batch * L * 64  # one head block's dB (or dC) partial sums
    r256 = lambda v: (v + 255) // 256 * 256
    rest = n.value - 2 * r256(nhb * part)
    # the rest of the workspace does not depend on the head blocks
    nc = (L + Q - 1) // Q
    E = 64 * 64
    Lp = nc * Q
    want_rest = (2 * r256(batch * H * Lp * 4) + (2 if nc <= 32 else 3) * r256(batch * nc * H * E * 4) +
                 3 * r256(batch * nc * H * E * 2) +
                 r256(batch * H * nc * (8 if nc <= 32 else 4) * 4) + r256(batch * H * Lp * 4) +
                 4 * r256(batch * H * Lp * 4) +
                 2 * r256(batch * nc * H * 4))
    assert rest == want_rest, (rest, want_rest)


def test_ssd_workspace_size():
    d, p = _ssd(batch=4, L=4096, H=80, Q=256)
    n = ssm.ssd_chunk_workspace_size(d)
    nc = 16
    want = 2 * 4 * 80 * 4096 * 4 + 4 * nc * 80 * 64 * 64 * 4 + 4 * nc * 80 * 64 * 64 * 2
    assert n == want
    assert ssm.lib().ssm_ssd_chunk_fwd(ctypes.byref(d), ctypes.byref(p), None, 0, None) == ssm.SSM_ERR_WORKSPACE


def _upd(batch=3, D=8, N=16, io="bf16", flags=0, **over):
    ts = {"x": T((batch, D), io, ptr=1 << 36), "delta": T((batch, D), io, ptr=2 << 36),
          "A": T((D, N), ptr=3 << 36), "B": T((batch, N), io, ptr=4 << 36), "C": T((batch, N), io, ptr=5 << 36),
          "D": T((D,), ptr=6 << 36), "z": T((batch, D), io, ptr=7 << 36), "y": T((batch, D), io, ptr=8 << 36),
          "state": T((batch, D, N), ptr=9 << 36), "delta_bias": T((D,), ptr=10 << 36)}
    ts.update(over)
    d = ssm.UpdateDesc()
    d.batch, d.dim, d.dstate, d.flags = batch, D, N, flags
    p = ssm.UpdatePtrs()
    for k, t in ts.items():
        setattr(d, k, _td(t))
        setattr(p, k, None if t is None else t.ptr)
    return d, p


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(p, "state", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "z", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(d, "batch", 0), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(d, "dstate", 65), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_HAS_H0), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_WANT_HLAST), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.x, "dtype", 2), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.state, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(d.C, "dtype", 0), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.B.shape.__setitem__(1, 8), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(d.x, "ndim", 3), ssm.SSM_ERR_SHAPE),
    (lambda d, p: d.state.stride.__setitem__(2, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: d.z.stride.__setitem__(1, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: d.y.stride.__setitem__(0, 0), ssm.SSM_ERR_STRIDE),
    (lambda d, p: setattr(p, "state", (9 << 36) + 2), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "y", p.x), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "state", p.A + 64), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "y", p.state + 4), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(d, "flags", d.flags & ~ssm.SSM_DELTA_SOFTPLUS), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(p, "delta_bias", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(d.delta_bias, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(p, "state", p.delta_bias), ssm.SSM_ERR_ALIAS),
])
def test_update_validation(mutate, status):
    d, p = _upd(flags=ssm.SSM_HAS_Z | ssm.SSM_HAS_D | ssm.SSM_DELTA_SOFTPLUS | ssm.SSM_HAS_DELTA_BIAS)
    mutate(d, p)
    assert ssm.lib().ssm_selective_state_update(ctypes.byref(d), ctypes.byref(p), None) == status


def test_update_null_descriptor():
    d, p = _upd()
    assert ssm.lib().ssm_selective_state_update(None, ctypes.byref(p), None) == ssm.SSM_ERR_NULL
    assert ssm.lib().ssm_selective_state_update(ctypes.byref(d), None, None) == ssm.SSM_ERR_NULL


def _conv(batch=2, L=40, D=12, W=4, io="bf16", flags=ssm.SSM_HAS_BIAS | ssm.SSM_SILU, **over):
    ts = {"x": T((batch, L, D), io, ptr=1 << 36), "weight": T((D, W), ptr=2 << 36), "bias": T((D,), ptr=3 << 36),
          "y": T((batch, L, D), io, ptr=4 << 36)}
    ts.update(over)
    d = ssm.ConvDesc()
    d.batch, d.seqlen, d.dim, d.width, d.flags = batch, L, D, W, flags
    p = ssm.ConvPtrs()
    for k, t in ts.items():
        setattr(d, k, _td(t))
        setattr(p, k, None if t is None else t.ptr)
    return d, p


@pytest.mark.parametrize("mutate,status", [
    (lambda d, p: setattr(p, "x", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(p, "bias", None), ssm.SSM_ERR_NULL),
    (lambda d, p: setattr(d, "seqlen", 0), ssm.SSM_ERR_SHAPE),
    (lambda d, p: setattr(d, "width", 9), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d, "flags", d.flags | ssm.SSM_HAS_Z), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.x, "dtype", 2), ssm.SSM_ERR_UNSUPPORTED),
    (lambda d, p: setattr(d.weight, "dtype", 1), ssm.SSM_ERR_DTYPE),
    (lambda d, p: setattr(d.y, "dtype", 2), ssm.SSM_ERR_DTYPE),
    (lambda d, p: d.weight.shape.__setitem__(1, 3), ssm.SSM_ERR_SHAPE),
    (lambda d, p: d.x.stride.__setitem__(2, 2), ssm.SSM_ERR_STRIDE),
    (lambda d, p: d.y.stride.__setitem__(1, 0), ssm.SSM_ERR_STRIDE),
    (lambda d, p: setattr(p, "x", (1 << 36) + 1), ssm.SSM_ERR_ALIGN),
    (lambda d, p: setattr(p, "y", p.x), ssm.SSM_ERR_ALIAS),
    (lambda d, p: setattr(p, "y", p.bias - 8), ssm.SSM_ERR_ALIAS),
])
def test_conv_validation(mutate, status):
    d, p = _conv()
    mutate(d, p)
    assert ssm.lib().ssm_causal_conv1d_fwd(ctypes.byref(d), ctypes.byref(p), None) == status


def test_conv_null_descriptor():
    d, p = _conv()
    assert ssm.lib().ssm_causal_conv1d_fwd(None, ctypes.byref(p), None) == ssm.SSM_ERR_NULL


@pytest.mark.parametrize("key,bad", [("A_cum", lambda t: t[..., :-1]), ("beta", lambda t: t.double()),
                                     ("states", lambda t: t.transpose(3, 4))])
def test_ssd_bwd_fwd_buffers_checked_by_the_binding(key, bad):
    # the library sees bare pointers for the forward's intermediates, so the
    # binding checks their shape, dtype and layout before any call
    torch = _torch
    batch, L, H, P, N, Q = 1, 100, 4, 64, 64, 64
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    x, dy, delta, B, C = bf(batch, L, H, P), bf(batch, L, H, P), bf(batch, L, H), bf(batch, L, 1, N), bf(batch, L, 1, N)
    A = torch.zeros(H)
    fwd = {"A_cum": torch.zeros(batch, H, 128), "beta": torch.zeros(batch, H, 128),
           "states": torch.zeros(batch, 2, H, P, N)}
    fwd[key] = bad(fwd[key])
    with pytest.raises(ValueError, match=key):
        ssm.ssd_bwd(dy, x, delta, A, B, C, Q, fwd=fwd)


@pytest.mark.parametrize("where", ["A_cum", "states", "dx", "x"])
def test_ssd_bwd_workspace_may_not_overlap(where):
    # the backward writes its workspace: it may not overlap an input, an
    # output or the forward's intermediates it reads
    d, p = _ssd_bwd(flags=ssm.SSM_HAS_D | ssm.SSM_HAS_H0 | ssm.SSM_HAS_SSD_FWD)
    for k, v in _FWD.items():
        setattr(p, k, v)
    ws = getattr(p, where) + 256
    assert ssm.lib().ssm_ssd_bwd(ctypes.byref(d), ctypes.byref(p), ws, 1 << 40, None) == ssm.SSM_ERR_ALIAS


@pytest.mark.parametrize("key,value", [("chunk", 128), ("euler", True)])
def test_ssd_bwd_refuses_intermediates_of_another_forward(key, value):
    # ssd_chunk_fwd_train records the chunk size and the discretisation of
    # its intermediates; a backward with others would compute wrong gradients
    torch = _torch
    batch, L, H, P, N, Q = 1, 100, 4, 64, 64, 64
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    x, dy, delta, B, C = bf(batch, L, H, P), bf(batch, L, H, P), bf(batch, L, H), bf(batch, L, 1, N), bf(batch, L, 1, N)
    fwd = {"A_cum": torch.zeros(batch, H, 128), "beta": torch.zeros(batch, H, 128),
           "states": torch.zeros(batch, 2, H, P, N), "chunk": Q, "euler": False}
    fwd[key] = value
    with pytest.raises(ValueError, match=key):
        ssm.ssd_bwd(dy, x, delta, torch.zeros(H), B, C, Q, fwd=fwd)
