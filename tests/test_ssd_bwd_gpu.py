"""GPU parity of ssm_ssd_bwd (the SSD backward on bf16 matrix cores) against
the fp64 oracle backward (oracle.ssd_bwd).

Inputs and dy are bf16 (exact in the oracle), with 64, 128 and 256 states;
the kernels round the
intermediate matrices E, M, the chunk-entry states and their gradients to
bf16 as matrix-core operands and accumulate in fp32, so every gradient is
held to the bf16 bar rel-L2 <= 2e-2.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import banner, dev_tensor, host_f64, metrics

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_60_amd as ssm  # noqa: E402

REL = 2e-2


def _check(spec, seed=0, h0=False, dx_dtype=None, patch=None, from_fwd=False):
    banner("ssd bwd %s seed %d h0%d fwd%d" % (spec.name, seed, h0, from_fwd))
    inp = synth.ssd_inputs(spec, seed)
    if patch:
        patch(inp)
    dy = synth.fill((spec.batch, spec.seqlen, spec.nheads, spec.headdim), synth.Dist(synth.NORMAL, 0.0, 1.0),
                    "bf16", seed, 21)
    h0v = synth.state_input((spec.batch, spec.nheads, spec.headdim, spec.dstate), seed) if h0 else None
    g = {k: dev_tensor(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    A = dev_tensor(inp["A"], "f32")
    Dk = dev_tensor(inp["D"], "f32") if "D" in inp else None
    h0d = None if h0v is None else torch.from_numpy(h0v).cuda()
    saved = None
    if from_fwd:   # the backward reads the forward's A_cum, beta and chunk states
        _, _, saved = ssm.ssd_chunk_fwd_train(g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, D=Dk, h0=h0d,
                                              euler=spec.euler)
    got = ssm.ssd_bwd(dev_tensor(dy, "bf16"), g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, D=Dk,
                      h0=h0d, euler=spec.euler, dx_dtype=dx_dtype, fwd=saved)
    torch.cuda.synchronize()
    ref = oracle.ssd_bwd(inp, "bf16", dy, ngroups=spec.ngroups, euler=spec.euler,
                         h0=None if h0v is None else h0v.astype(np.float64))
    assert set(got) == set(ref), (set(got), set(ref))
    for k in sorted(ref):
        m = metrics(host_f64(got[k]), ref[k])
        print(k, m, flush=True)
        assert m["nan"] == 0, (k, m)
        assert m["rel_l2"] <= REL, (k, m)
    return got


def small(**kw):
    base = dict(batch=2, seqlen=300, nheads=4, chunk=64)
    base.update(kw)
    return synth.ssd_spec(synth.SSD2_7B, **base)


def test_ssd_bwd_small():
    _check(small(), 1)


@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("seqlen", [1, 63, 256, 300, 1000])
def test_ssd_bwd_chunks_and_ragged_lengths(chunk, seqlen):
    _check(small(seqlen=seqlen, chunk=chunk), 2)


@pytest.mark.parametrize("kw", [dict(ngroups=2), dict(ngroups=4, nheads=8), dict(has_D=False), dict(euler=True),
                                dict(nheads=13), dict(nheads=40, seqlen=130), dict(batch=1, nheads=1)],
                         ids=lambda kw: "_".join("%s%s" % i for i in sorted(kw.items())))
def test_ssd_bwd_flags_and_heads(kw):
    _check(small(**kw), 3)


@pytest.mark.parametrize("kw", [dict(dstate=128, chunk=64), dict(dstate=128, chunk=128), dict(dstate=128, chunk=256),
                                dict(dstate=256, chunk=64), dict(dstate=256, chunk=128),
                                dict(dstate=128, chunk=128, seqlen=1000, ngroups=2),
                                dict(dstate=256, chunk=64, seqlen=77, nheads=3)],
                         ids=lambda kw: "_".join("%s%s" % i for i in sorted(kw.items())))
def test_ssd_bwd_larger_states(kw):
    _check(small(**kw), 7)


def test_ssd_bwd_larger_states_h0():
    _check(small(dstate=128, chunk=128), 8, h0=True, dx_dtype=torch.float32)


def test_ssd_bwd_2_7b_n128_batch1():
    """The 2.7B-shaped layer with 128 states (chunk 128), one sequence of 4096
    steps, 80 heads: every gradient against the oracle."""
    _check(synth.ssd_spec(synth.SSD2_7B, batch=1, dstate=128, chunk=128), 9)


def test_ssd_bwd_h0_and_f32_dx():
    got = _check(small(chunk=128), 4, h0=True, dx_dtype=torch.float32)
    assert got["dx"].dtype == torch.float32


def test_ssd_bwd_zero_A_head():
    # A_h = 0: beta = delta and dbeta/dA = delta^2 / 2 (the series branch)
    def patch(inp):
        inp["A"][1] = 0.0
    _check(small(), 5, patch=patch)


def test_ssd_bwd_deterministic():
    spec = small(nheads=16, seqlen=600, chunk=128)
    a = _check(spec, 6)
    inp = synth.ssd_inputs(spec, 6)
    dy = synth.fill((spec.batch, spec.seqlen, spec.nheads, spec.headdim), synth.Dist(synth.NORMAL, 0.0, 1.0),
                    "bf16", 6, 21)
    g = {k: dev_tensor(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    b = ssm.ssd_bwd(dev_tensor(dy, "bf16"), g["x"], g["delta"], dev_tensor(inp["A"], "f32"), g["B"], g["C"],
                    spec.chunk, D=dev_tensor(inp["D"], "f32"))
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_ssd_bwd_2_7b_full():
    """The 2.7B-shaped layer (batch 4, L 4096, 80 heads x 64, N 64, chunk
    256): every gradient against the oracle at full size."""
    _check(synth.SSD2_7B, 0)


@pytest.mark.parametrize("kw,h0", [(dict(), True), (dict(seqlen=1000, chunk=256), False),
                                   (dict(ngroups=2, euler=True, chunk=128), False),
                                   (dict(dstate=128, chunk=128, seqlen=200), True),
                                   (dict(dstate=256, chunk=64, seqlen=130), False)])
def test_ssd_bwd_from_forward_intermediates(kw, h0):
    """With the forward's A_cum, beta and chunk states passed in
    (SSM_HAS_SSD_FWD): every gradient against the oracle, and equal bit for
    bit to the backward that recomputes them (the same kernels on the same
    values)."""
    spec = small(**kw)
    got = _check(spec, 7, h0=h0, from_fwd=True)
    ref = _check(spec, 7, h0=h0)
    for k in ref:
        assert torch.equal(got[k], ref[k]), k


def test_ssd_forward_by_steps_keeps_intermediates():
    """ssd_chunk_fwd_train runs the four steps: its y and h_last equal the
    one-call forward's, and its kept A_cum, beta and states are the steps'
    own outputs."""
    spec = small(seqlen=333, chunk=128)
    banner("ssd fwd train %s" % spec.name)
    inp = synth.ssd_inputs(spec, 8)
    g = {k: dev_tensor(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    A, Dk = dev_tensor(inp["A"], "f32"), dev_tensor(inp["D"], "f32")
    h0 = torch.from_numpy(synth.state_input((spec.batch, spec.nheads, spec.headdim, spec.dstate), 8)).cuda()
    y, hl, saved = ssm.ssd_chunk_fwd_train(g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, D=Dk, h0=h0,
                                           want_hlast=True)
    y1, hl1 = ssm.ssd_chunk_fwd(g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, D=Dk, h0=h0, want_hlast=True)
    A_cum, beta = ssm.ssd_chunk_cumsum(g["x"], g["delta"], A, g["B"], g["C"], spec.chunk)
    states = ssm.ssd_chunk_state(g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, A_cum, beta)
    torch.cuda.synchronize()
    assert torch.equal(y, y1) and torch.equal(hl, hl1)
    L = spec.seqlen
    nc = -(-L // spec.chunk)
    assert torch.equal(saved["states"], states)
    # A_cum and beta are specified for the first seqlen steps of each row
    for k, v in (("A_cum", A_cum), ("beta", beta)):
        assert torch.equal(saved[k][..., :L], v[..., :L]), k
    assert saved["A_cum"].shape == (spec.batch, spec.nheads, nc * spec.chunk)


def test_ssd_bwd_fwd_shape_checked():
    spec = small()
    inp = synth.ssd_inputs(spec, 9)
    g = {k: dev_tensor(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    A = dev_tensor(inp["A"], "f32")
    _, _, saved = ssm.ssd_chunk_fwd_train(g["x"], g["delta"], A, g["B"], g["C"], spec.chunk)
    saved["states"] = saved["states"][:, :-1]   # one chunk short
    with pytest.raises(ValueError):
        ssm.ssd_bwd(g["x"], g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, fwd=saved)


def test_ssd_bwd_from_forward_2_7b_full_equals_recompute():
    """At the 2.7B-shaped layer's full size, in the configuration the bench
    times: the backward reading the forward's intermediates equals, bit for
    bit, the recomputing backward (whose gradients the full-size oracle test
    above checks)."""
    spec = synth.SSD2_7B
    banner("ssd bwd from fwd %s" % spec.name)
    inp = synth.ssd_inputs(spec, 0)
    dy = dev_tensor(synth.fill((spec.batch, spec.seqlen, spec.nheads, spec.headdim),
                               synth.Dist(synth.NORMAL, 0.0, 1.0), "bf16", 0, 21), "bf16")
    g = {k: dev_tensor(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    A, Dk = dev_tensor(inp["A"], "f32"), dev_tensor(inp["D"], "f32")
    del inp
    _, _, saved = ssm.ssd_chunk_fwd_train(g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, D=Dk)
    a = ssm.ssd_bwd(dy, g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, D=Dk, fwd=saved)
    b = ssm.ssd_bwd(dy, g["x"], g["delta"], A, g["B"], g["C"], spec.chunk, D=Dk)
    torch.cuda.synchronize()
    assert set(a) == set(b)
    for k in b:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("seqlen", [1024, 1040, 2048, 2100])
def test_ssd_bwd_state_pass_chunk_counts(seqlen):
    """Chunk counts on both sides of the state pass's register-history limits
    (16 and 32 chunks kept in registers, more by the kernel that keeps them
    in memory): 16, 17, 32 and 33 chunks of 64 steps, with h0 (dh0 is the
    gradient carried out of the first chunk)."""
    _check(small(batch=1, nheads=2, seqlen=seqlen, chunk=64), 10, h0=True)
