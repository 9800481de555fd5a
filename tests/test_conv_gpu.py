"""GPU parity of ssm_causal_conv1d_fwd (causal depthwise conv + bias + SiLU)
against the fp64 oracle.

fp32 outputs (from fp32 or bf16 inputs, both exact in the oracle) meet
rel-L2 <= 1e-5 and max-abs <= 1e-4; bf16 outputs meet the bf16 bound.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import assert_close, banner, dev_tensor, host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import selective_state_space_60_amd as ssm  # noqa: E402


def _run(spec, inp, y_dtype=None, x=None):
    xd = dev_tensor(inp["x"], spec.io) if x is None else x
    w = dev_tensor(inp["weight"], "f32")
    b = dev_tensor(inp["bias"], "f32") if "bias" in inp else None
    y = ssm.causal_conv1d(xd, w, b, silu=spec.silu, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y


def _check(spec, seed=0):
    banner("conv %s seed %d" % (spec.name, seed))
    inp = synth.conv_inputs(spec, seed)
    ref = oracle.causal_conv1d(inp["x"], inp["weight"], spec.io, inp.get("bias"), silu=spec.silu)
    y = _run(spec, inp)
    assert_close(host_f64(y), ref, spec.io, spec.name + " y")
    y32 = _run(spec, inp, y_dtype=torch.float32)
    assert_close(host_f64(y32), ref, "f32", spec.name + " y (fp32 out)")


def test_conv_2_8b_full():
    """The Mamba-2.8B layer's width-4 conv (4 x 4096 x 5120, bf16), every output."""
    _check(synth.CONV2_8B, 0)


EDGE = [
    # (batch, L, D, W, io, bias, silu)
    (1, 1, 4, 4, "f32", True, True),
    (2, 3, 8, 4, "bf16", True, True),      # L < W
    (1, 33, 12, 1, "f32", False, True),
    (2, 95, 1028, 2, "bf16", True, False),  # two channel blocks, ragged runs
    (3, 64, 30, 3, "f32", True, True),      # D % 4 != 0: one channel per lane
    (1, 129, 37, 5, "bf16", False, True),
    (2, 70, 96, 8, "f32", True, True),
    (1, 100, 5120, 4, "bf16", True, True),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "b%d_l%d_d%d_w%d_%s_bias%d_silu%d" % c)
def test_conv_edges(case):
    batch, L, D, W, io, bias, silu = case
    spec = synth.conv_spec(synth.CONV2_8B, batch=batch, seqlen=L, dim=D, width=W, io=io, has_bias=bias, silu=silu)
    _check(spec, 3)


def test_conv_strided_input_view():
    """x as a view into a wider (batch, L, 2*D) buffer (the in_proj output holds x and z side by side)."""
    spec = synth.conv_spec(synth.CONV2_8B, batch=2, seqlen=77, dim=64)
    inp = synth.conv_inputs(spec, 4)
    banner("conv strided")
    xz = torch.zeros((2, 77, 128), dtype=torch.bfloat16, device="cuda")
    xz[:, :, :64] = dev_tensor(inp["x"], "bf16")
    y = _run(spec, inp, y_dtype=torch.float32, x=xz[:, :, :64])
    ref = oracle.causal_conv1d(inp["x"], inp["weight"], "bf16", inp["bias"])
    assert_close(host_f64(y), ref, "f32", "conv strided")


def test_conv_deterministic():
    spec = synth.conv_spec(synth.CONV2_8B, batch=2, seqlen=300, dim=256)
    inp = synth.conv_inputs(spec, 5)
    banner("conv determinism")
    assert torch.equal(_run(spec, inp), _run(spec, inp))
