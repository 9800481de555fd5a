"""GPU parity of ssm_selective_state_update (one recurrent decode step)
against the fp64 oracle.

T decode steps chained on one in-place state must reproduce the oracle's
selective scan over the same T steps started from the same h0: every step's
y and the final state.  fp32 inputs: rel-L2 <= 1e-5, max-abs <= 1e-4.  bf16
inputs are exact bf16 values and the state is fp32, so the state and an fp32
y meet the fp32 bound too; a bf16 y meets the bf16 bound.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import assert_close, banner, dev_tensor, host_f64, metrics

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_60_amd as ssm  # noqa: E402


def _upload(spec, inp):
    io = spec.io
    d = {k: dev_tensor(inp[k], io) for k in ("x", "delta", "B", "C")}
    d["A"] = dev_tensor(inp["A"], "f32")
    d["D"] = dev_tensor(inp["D"], "f32") if "D" in inp else None
    d["z"] = dev_tensor(inp["z"], io) if "z" in inp else None
    return d


def _decode(spec, inp, h0, y_dtype=None):
    """Run the L steps of `inp` one decode call at a time on a device state.
    Returns (y (batch, L, D) on host as f64, final state on device)."""
    g = _upload(spec, inp)
    state = torch.from_numpy(np.ascontiguousarray(h0, np.float32)).cuda()
    ys = []
    for t in range(spec.seqlen):
        z = None if g["z"] is None else g["z"][:, t]
        y = ssm.selective_state_update(state, g["x"][:, t], g["delta"][:, t], g["A"], g["B"][:, t],
                                       g["C"][:, t], D=g["D"], z=z, euler=spec.euler, y_dtype=y_dtype)
        ys.append(y)
    torch.cuda.synchronize()
    return np.stack([host_f64(y) for y in ys], axis=1), state


def _check(spec, seed, y_dtype=None, h0=None):
    banner("update %s seed %d" % (spec.name, seed))
    inp = synth.scan_inputs(spec, seed)
    if h0 is None:
        h0 = synth.state_input((spec.batch, spec.dim, spec.dstate), seed)
    y, state = _decode(spec, inp, h0, y_dtype)
    yr, hr = oracle.selective_scan(inp, spec.io, euler=spec.euler, h0=h0.astype(np.float64))
    y_io = "f32" if (spec.io == "f32" or y_dtype == torch.float32) else "bf16"
    assert_close(y, yr, y_io, spec.name + " y")
    assert_close(host_f64(state), hr, "f32", spec.name + " state")


def test_decode_2_8b_one_step_full():
    """The Mamba-2.8B-shaped decode step (64 sequences x 5120 channels x 16
    states), every output, bf16 y and fp32 y."""
    _check(synth.DECODE2_8B, 0)
    _check(synth.DECODE2_8B, 1, y_dtype=torch.float32)


EDGE = [
    # (batch, T, D, N, io, has_z, has_D, euler)
    (1, 1, 1, 1, "f32", False, False, False),
    (1, 5, 4, 4, "f32", False, True, False),
    (2, 8, 33, 16, "f32", True, True, False),
    (3, 6, 37, 20, "f32", True, False, False),
    (2, 4, 40, 32, "f32", True, True, False),
    (1, 4, 48, 64, "f32", True, True, False),
    (2, 7, 96, 8, "f32", False, False, True),
    (2, 7, 100, 16, "bf16", True, True, False),
    (2, 5, 96, 16, "bf16", True, True, True),
    (1, 3, 48, 64, "bf16", True, True, False),
    (7, 3, 130, 6, "f32", True, True, False),
    (6, 3, 300, 64, "bf16", True, True, False),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "b%d_t%d_d%d_n%d_%s_z%d_D%d_e%d" % c)
def test_chained_steps_equal_the_scan(case):
    batch, T, D, N, io, z, Dk, eu = case
    base = synth.TINY if io == "f32" else synth.MAMBA130M
    spec = synth.scan_spec(base, batch=batch, seqlen=T, dim=D, dstate=N, io=io, has_z=z, has_D=Dk, euler=eu,
                           A=synth.Dist(synth.NEG_EXP_UNIFORM, -1.0, 1.0))
    _check(spec, 3)
    if io == "bf16":
        _check(spec, 4, y_dtype=torch.float32)


def test_zero_state_and_zero_A():
    """h0 = 0 (a fresh sequence) and A = 0 entries (Bbar = delta * B)."""
    spec = synth.scan_spec(synth.TINY, batch=2, seqlen=6, dim=20, dstate=8, has_z=True)
    inp = synth.scan_inputs(spec, 9)
    inp["A"][3, :] = 0.0
    inp["A"][7, 2] = 0.0
    _check(spec, 9, h0=np.zeros((2, 20, 8), np.float32))


def test_matches_the_scan_kernel():
    """Decode steps after a prefill by the scan kernel continue its state."""
    spec = synth.scan_spec(synth.MAMBA130M, batch=2, seqlen=40, dim=96, dstate=16)
    inp = synth.scan_inputs(spec, 11)
    banner("update after scan prefill")
    g = _upload(spec, inp)
    L1 = 33
    _, hl = ssm.selective_scan_fwd(g["x"][:, :L1], g["delta"][:, :L1], g["A"], g["B"][:, :L1], g["C"][:, :L1],
                                   D=g["D"], z=g["z"][:, :L1], want_hlast=True, y_dtype=torch.float32)
    ys = []
    for t in range(L1, spec.seqlen):
        ys.append(ssm.selective_state_update(hl, g["x"][:, t], g["delta"][:, t], g["A"], g["B"][:, t],
                                             g["C"][:, t], D=g["D"], z=g["z"][:, t], y_dtype=torch.float32))
    torch.cuda.synchronize()
    yr, hr = oracle.selective_scan(inp, "bf16")
    y = np.stack([host_f64(v) for v in ys], axis=1)
    assert_close(y, yr[:, L1:], "f32", "decode after prefill y")
    assert_close(host_f64(hl), hr, "f32", "decode after prefill state")


def test_broadcast_A_and_strided_views():
    """A with stride 0 over channels; x/delta/z/y/B/C as strided views."""
    spec = synth.scan_spec(synth.TINY, batch=3, seqlen=1, dim=50, dstate=16, has_z=True)
    inp = synth.scan_inputs(spec, 7)
    inp["A"] = np.broadcast_to(inp["A"][:1].copy(), (50, 16)).copy()
    h0 = synth.state_input((3, 50, 16), 7)
    banner("update strided")
    g = _upload(spec, inp)
    wide = {}
    for k in ("x", "delta", "z"):
        buf = torch.zeros((3, 64), dtype=torch.float32, device="cuda")
        buf[:, 8:58] = g[k][:, 0]
        wide[k] = buf[:, 8:58]
    BC = torch.zeros((3, 2, 16), dtype=torch.float32, device="cuda")
    BC[:, 0], BC[:, 1] = g["B"][:, 0], g["C"][:, 0]
    ybuf = torch.full((3, 70), 7.0, dtype=torch.float32, device="cuda")
    A0 = g["A"][:1].expand(50, 16)
    state = torch.from_numpy(h0).cuda()
    ssm.selective_state_update(state, wide["x"], wide["delta"], A0, BC[:, 0], BC[:, 1], D=g["D"], z=wide["z"],
                               y=ybuf[:, 10:60])
    torch.cuda.synchronize()
    yr, hr = oracle.selective_scan(inp, "f32", h0=h0.astype(np.float64))
    assert_close(host_f64(ybuf[:, 10:60]), yr[:, 0], "f32", "strided y")
    assert_close(host_f64(state), hr, "f32", "strided state")
    assert torch.all(ybuf[:, :10] == 7.0) and torch.all(ybuf[:, 60:] == 7.0)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_non_unit_state_strides(io):
    """B, C with stride 2 along the state and A stored transposed (the
    kernel's scalar-load variant), and an odd batch."""
    base = synth.TINY if io == "f32" else synth.MAMBA130M
    spec = synth.scan_spec(base, batch=5, seqlen=2, dim=72, dstate=16, io=io, has_z=True, has_D=True,
                           A=synth.Dist(synth.NEG_EXP_UNIFORM, -1.0, 1.0))
    inp = synth.scan_inputs(spec, 12)
    h0 = synth.state_input((5, 72, 16), 12)
    banner("update non-unit strides %s" % io)
    g = _upload(spec, inp)
    dt = torch.float32 if io == "f32" else torch.bfloat16
    At = g["A"].t().contiguous().t()  # (72, 16) with strides (1, 72)
    assert At.stride(1) != 1
    state = torch.from_numpy(h0).cuda()
    ys = []
    for t in range(2):
        Bw = torch.zeros((5, 32), dtype=dt, device="cuda")
        Cw = torch.zeros((5, 32), dtype=dt, device="cuda")
        Bw[:, ::2], Cw[:, ::2] = g["B"][:, t], g["C"][:, t]
        ys.append(ssm.selective_state_update(state, g["x"][:, t], g["delta"][:, t], At, Bw[:, ::2], Cw[:, ::2],
                                             D=g["D"], z=g["z"][:, t], y_dtype=torch.float32))
    torch.cuda.synchronize()
    yr, hr = oracle.selective_scan(inp, io, h0=h0.astype(np.float64))
    assert_close(np.stack([host_f64(v) for v in ys], axis=1), yr, "f32", "non-unit strides y")
    assert_close(host_f64(state), hr, "f32", "non-unit strides state")


def test_deterministic():
    spec = synth.scan_spec(synth.DECODE2_8B, batch=4, dim=1024)
    inp = synth.scan_inputs(spec, 2)
    h0 = synth.state_input((4, 1024, 16), 2)
    banner("update determinism")
    y1, s1 = _decode(spec, inp, h0)
    y2, s2 = _decode(spec, inp, h0)
    assert np.array_equal(y1, y2) and torch.equal(s1, s2)


def test_nan_stays_in_its_channel():
    spec = synth.scan_spec(synth.TINY, batch=1, seqlen=3, dim=40, dstate=16, has_z=False)
    inp = synth.scan_inputs(spec, 6)
    inp["x"][0, 1, 5] = np.nan
    banner("update NaN")
    y, state = _decode(spec, inp, np.zeros((1, 40, 16), np.float32))
    assert np.all(np.isfinite(y[0, 0]))
    assert np.all(np.isnan(y[0, 1:, 5]))
    assert np.all(np.isfinite(np.delete(y, 5, axis=2)))
    st = host_f64(state)
    assert np.all(np.isnan(st[0, 5])) and np.all(np.isfinite(np.delete(st, 5, axis=1)))


@pytest.mark.parametrize("io,N,strided", [("f32", 16, False), ("bf16", 16, False), ("f32", 6, False),
                                           ("bf16", 16, True)])
def test_delta_softplus(io, N, strided):
    """delta <- softplus(delta + bias), vector and generic paths, chained
    steps against the oracle's scan with the same transform."""
    base = synth.TINY if io == "f32" else synth.MAMBA130M
    spec = synth.scan_spec(base, batch=3, seqlen=4, dim=72, dstate=N, io=io, has_z=True, has_D=True,
                           A=synth.Dist(synth.NEG_EXP_UNIFORM, -1.0, 1.0), delta=synth.Dist(synth.NORMAL, 0.0, 1.0))
    inp = synth.scan_inputs(spec, 15)
    db = synth.delta_bias_input(72, 15)
    h0 = synth.state_input((3, 72, N), 15)
    banner("update softplus %s N%d strided%d" % (io, N, strided))
    g = _upload(spec, inp)
    A = g["A"].t().contiguous().t() if strided else g["A"]
    state = torch.from_numpy(h0).cuda()
    dbd = torch.from_numpy(db).cuda()
    ys = []
    for t in range(4):
        ys.append(ssm.selective_state_update(state, g["x"][:, t], g["delta"][:, t], A, g["B"][:, t], g["C"][:, t],
                                             D=g["D"], z=g["z"][:, t], y_dtype=torch.float32, delta_softplus=True,
                                             delta_bias=dbd))
    torch.cuda.synchronize()
    yr, hr = oracle.selective_scan(inp, io, h0=h0.astype(np.float64), delta_softplus=True, delta_bias=db)
    assert_close(np.stack([host_f64(v) for v in ys], axis=1), yr, "f32", "update softplus y")
    assert_close(host_f64(state), hr, "f32", "update softplus state")
