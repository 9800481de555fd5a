"""GPU parity of the SSD chunked path (ssm_ssd_chunk_fwd and its four steps)
against the fp64 oracle.

y and h_last are compared with the oracle's expanded recurrence (bf16 inputs,
fp32 state: rel-L2 <= 2e-2).  Each step's intermediate is compared with the
oracle's chunked algorithm on the same inputs: A_cum and beta (fp32 on the
GPU) to 1e-5 relative, the chunk states and chunk-entry states (bf16 matrix
cores) to the bf16 bound.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import BF16_REGRESSION, assert_close, assert_tiles, banner, dev_tensor, host_f64, metrics

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_60_amd as ssm  # noqa: E402


def _upload(inp):
    d = {k: dev_tensor(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    d["A"] = dev_tensor(inp["A"], "f32")
    d["D"] = dev_tensor(inp["D"], "f32") if "D" in inp else None
    return d


def _run(spec, inp, h0=None, want_hlast=True, y_dtype=None):
    g = _upload(inp)
    h0d = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, np.float32)).cuda()
    y, hl = ssm.ssd_chunk_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], spec.chunk, D=g["D"], h0=h0d,
                              euler=spec.euler, want_hlast=want_hlast, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y, hl


def _check(spec, seed=0, h0=None, rows=None):
    banner("ssd %s seed %d" % (spec.name, seed))
    inp = synth.ssd_inputs(spec, seed)
    y, hl = _run(spec, inp, h0=h0)
    h064 = None if h0 is None else np.asarray(h0, np.float32).astype(np.float64)
    if rows is None:
        yr, hr = oracle.ssd(inp, "bf16", ngroups=spec.ngroups, euler=spec.euler, h0=h064)
        assert_close(host_f64(y), yr, "bf16", spec.name + " y")
        assert_close(host_f64(hl), hr, "bf16", spec.name + " h_last")
    else:
        yr, hr = oracle.ssd(inp, "bf16", ngroups=spec.ngroups, euler=spec.euler, h0=h064, rows=rows)
        HP = spec.nheads * spec.headdim
        b, hh, pp = rows // HP, (rows % HP) // spec.headdim, rows % spec.headdim
        yg = y[torch.as_tensor(b), :, torch.as_tensor(hh), torch.as_tensor(pp)]
        assert_close(host_f64(yg), yr, "bf16", spec.name + " y (sampled rows)")
        hg = hl[torch.as_tensor(b), torch.as_tensor(hh), torch.as_tensor(pp), :]
        assert_close(host_f64(hg), hr, "bf16", spec.name + " h_last (sampled rows)")
    return y


def small(**kw):
    base = dict(batch=2, seqlen=300, nheads=4, chunk=64)
    base.update(kw)
    return synth.ssd_spec(synth.SSD2_7B, **base)


def test_ssd_2_7b_full():
    """The 2.7B-shaped layer (batch 4, L 4096, 80 heads x 64, N 64, chunk 256)
    against the expanded recurrence, every output: the bf16 bar, then the
    regression bars on the whole output and on every (batch, chunk, head)
    tile."""
    s = synth.SSD2_7B
    y = _check(s, 0)
    yr, _ = oracle.ssd(synth.ssd_inputs(s, 0), "bf16", ngroups=s.ngroups)
    yh = host_f64(y)
    m = metrics(yh, yr)
    assert m["rel_l2"] <= BF16_REGRESSION["ssd"], m
    assert_tiles(yh, yr, (1, s.chunk, 1, s.headdim), 2e-2, s.name + " y")


@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("seqlen", [1, 63, 256, 300, 1000])
def test_chunk_sizes_and_ragged_lengths(chunk, seqlen):
    _check(small(seqlen=seqlen, chunk=chunk), 1)


@pytest.mark.parametrize("ngroups", [2, 4])
def test_groups(ngroups):
    _check(small(nheads=8, ngroups=ngroups, seqlen=333), 2)


def test_h0_and_euler_and_no_D():
    spec = small(seqlen=400, chunk=128)
    h0 = synth.state_input((2, 4, 64, 64), 3)
    _check(spec, 3, h0=h0)
    _check(synth.ssd_spec(spec, euler=True), 4)
    _check(synth.ssd_spec(spec, has_D=False), 5)


def test_fp32_output():
    spec = small(seqlen=200)
    inp = synth.ssd_inputs(spec, 6)
    banner("ssd f32 y")
    y, _ = _run(spec, inp, y_dtype=torch.float32)
    assert y.dtype == torch.float32
    yr, _ = oracle.ssd(inp, "bf16")
    assert_close(host_f64(y), yr, "bf16", "ssd fp32 y")


def test_steps_against_chunked_reference():
    """Each of the four steps against the oracle's chunked algorithm."""
    spec = small(seqlen=300, chunk=128, nheads=6, ngroups=2)
    inp = synth.ssd_inputs(spec, 7)
    h0 = synth.state_input((2, 6, 64, 64), 7)
    banner("ssd steps")
    g = _upload(inp)
    args = (g["x"], g["delta"], g["A"], g["B"], g["C"], spec.chunk)
    A_cum, beta = ssm.ssd_chunk_cumsum(*args)
    states = ssm.ssd_chunk_state(*args, A_cum, beta)
    h0d = torch.from_numpy(h0).cuda()
    S_in, hl = ssm.ssd_state_passing(*args, A_cum, states, h0=h0d, want_hlast=True)
    y = ssm.ssd_chunk_scan(*args, A_cum, beta, S_in, D=g["D"])
    torch.cuda.synchronize()
    ref = oracle.ssd_chunked(inp, "bf16", spec.chunk, ngroups=spec.ngroups, h0=h0.astype(np.float64))
    L = spec.seqlen
    m = metrics(host_f64(A_cum)[:, :, :L], ref["A_cum"])
    assert m["rel_l2"] < 1e-6, m
    m = metrics(host_f64(beta)[:, :, :L], ref["beta"])
    assert m["rel_l2"] < 1e-6, m
    # padded steps past L: no input, flat cumulative decay
    assert torch.all(beta[:, :, L:] == 0)
    assert_close(host_f64(states), ref["S_loc"], "bf16", "chunk states")
    assert_close(host_f64(S_in), ref["S_in"], "bf16", "chunk-entry states")
    assert_close(host_f64(hl), ref["h_last"], "bf16", "h_last")
    assert_close(host_f64(y), ref["y"], "bf16", "y")


def test_deterministic():
    spec = small(seqlen=500)
    inp = synth.ssd_inputs(spec, 8)
    banner("ssd determinism")
    y1, h1 = _run(spec, inp)
    y2, h2 = _run(spec, inp)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_strided_heads_view():
    """x as a view into a wider (batch, L, H+2, P) buffer (16-byte aligned rows)."""
    spec = small(seqlen=150)
    inp = synth.ssd_inputs(spec, 9)
    g = _upload(inp)
    wide = torch.zeros((2, 150, 6, 64), dtype=torch.bfloat16, device="cuda")
    wide[:, :, 1:5] = g["x"]
    xv = wide[:, :, 1:5]
    banner("ssd strided")
    y, _ = ssm.ssd_chunk_fwd(xv, g["delta"], g["A"], g["B"], g["C"], spec.chunk, D=g["D"])
    torch.cuda.synchronize()
    yr, _ = oracle.ssd(inp, "bf16")
    assert_close(host_f64(y), yr, "bf16", "ssd strided")


@pytest.mark.parametrize("chunk,y_dtype", [(64, None), (128, None), (256, None), (256, torch.float32)])
def test_strided_y_view_keeps_its_neighbours(chunk, y_dtype):
    """y as a view into a wider (batch, L, H+2, P) buffer filled with a
    sentinel, the sequence ending inside a chunk: the outputs (bf16 rows are
    stored 16 bytes a lane after lane swaps) land in the view, and the heads
    on either side and the rows after L keep the sentinel."""
    spec = small(seqlen=301, chunk=chunk)
    inp = synth.ssd_inputs(spec, 11)
    g = _upload(inp)
    H = spec.nheads
    dt = y_dtype or torch.bfloat16
    wide = torch.full((2, 303, H + 2, 64), 7.0, dtype=dt, device="cuda")
    yv = wide[:, :301, 1:H + 1]
    banner("ssd strided y chunk %d %s" % (chunk, dt))
    y, _ = ssm.ssd_chunk_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], spec.chunk, D=g["D"], y=yv)
    torch.cuda.synchronize()
    yr, _ = oracle.ssd(inp, "bf16")
    assert_close(host_f64(yv), yr, "bf16", "ssd strided y")
    assert bool((wide[:, :, 0] == 7.0).all()) and bool((wide[:, :, H + 1] == 7.0).all())
    assert bool((wide[:, 301:] == 7.0).all())


@pytest.mark.parametrize("dstate,chunk", [(128, 64), (128, 128), (128, 256), (256, 64), (256, 128)])
def test_larger_states(dstate, chunk):
    """N = 128 and 256 states (every supported chunk size), ragged length,
    grouped B/C, h0 and h_last, against the expanded recurrence."""
    spec = small(seqlen=333, chunk=chunk, nheads=4, ngroups=2, dstate=dstate)
    h0 = synth.state_input((2, 4, 64, dstate), 11)
    _check(spec, 11, h0=h0)


def test_larger_states_steps():
    """Each step's intermediate against the chunked reference at N = 256."""
    spec = small(seqlen=200, chunk=64, nheads=2, dstate=256)
    inp = synth.ssd_inputs(spec, 12)
    banner("ssd steps N256")
    g = _upload(inp)
    args = (g["x"], g["delta"], g["A"], g["B"], g["C"], spec.chunk)
    A_cum, beta = ssm.ssd_chunk_cumsum(*args)
    states = ssm.ssd_chunk_state(*args, A_cum, beta)
    S_in, hl = ssm.ssd_state_passing(*args, A_cum, states, want_hlast=True)
    y = ssm.ssd_chunk_scan(*args, A_cum, beta, S_in, D=g["D"])
    torch.cuda.synchronize()
    ref = oracle.ssd_chunked(inp, "bf16", spec.chunk)
    assert_close(host_f64(states), ref["S_loc"], "bf16", "chunk states N256")
    assert_close(host_f64(S_in), ref["S_in"], "bf16", "chunk-entry states N256")
    assert_close(host_f64(hl), ref["h_last"], "bf16", "h_last N256")
    assert_close(host_f64(y), ref["y"], "bf16", "y N256")


def _scale_bf16(bits, k):
    """bf16 bit patterns times 2**k (exact: the exponent field moves by k;
    zeros stay zero)."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    e = (b >> 7) & 0xFF
    assert np.all((e == 0) | ((e + k > 0) & (e + k < 255))), "scaled out of the normal range"
    return np.where(e == 0, b, b + (k << 7)).astype(np.uint16)


@pytest.mark.parametrize("kb,kc", [(10, 9), (-20, -20)])
@pytest.mark.parametrize("kw", [dict(chunk=256), dict(chunk=128, dstate=128), dict(chunk=64)],
                         ids=lambda kw: "_".join("%s%s" % i for i in sorted(kw.items())))
def test_magnitudes_of_B_and_C(kw, kb, kc):
    """B and C times powers of two far from 1: y (no D skip) scales by exactly
    2**(kb + kc) and h_last by 2**kb, bit for bit -- every step is
    scale-equivariant, including chunk_scan's fp16 copy of C B^T, whose own
    power-of-two scale follows max|B| max|C| (no tile may overflow fp16 or
    fall into its subnormals) -- and y still meets the oracle."""
    spec = small(seqlen=600, has_D=False, **kw)
    inp = synth.ssd_inputs(spec, 11)
    y0, h0_ = _run(spec, inp)
    inp2 = dict(inp)
    inp2["B"] = _scale_bf16(inp["B"], kb)
    inp2["C"] = _scale_bf16(inp["C"], kc)
    banner("ssd magnitudes %s kb %d kc %d" % (spec.name, kb, kc))
    y1, h1 = _run(spec, inp2)
    assert torch.equal(y1.float(), y0.float() * 2.0 ** (kb + kc))
    assert torch.equal(h1, h0_ * 2.0 ** kb)
    yr, _ = oracle.ssd(inp2, "bf16", ngroups=spec.ngroups)
    assert_close(host_f64(y1), yr, "bf16", spec.name + " y, scaled B and C")
