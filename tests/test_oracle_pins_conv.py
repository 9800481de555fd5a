"""Pins of the oracle's causal convolution and its delta softplus.

The Mamba block (tildalice.io "Mamba 논문 리뷰", Mamba 블록 아키텍처 and the
SelectiveSSM listing) puts a per-channel Conv1D of width k in front of the
scan.  It pads k - 1 steps on the left and keeps the first L outputs, then
applies SiLU.  Its step size is the softplus of a projection carrying a bias.

Pins:
  C1  The listing's own definition, run by torch's float64 conv1d on the CPU:
      groups = channels, padding = k - 1, output cut back to L, then SiLU.
  C2  Per channel, numpy.convolve with the taps reversed: the listing's layer
      is a cross-correlation.
  C3  Impulse response (the taps, in order, delayed) and causality.
  S1  Softplus through the scan: with N = 1, A = 0, B = C = x = 1 and L = 1 the
      scan returns delta itself, so y = softplus(v).  Checked against ln 2 at 0,
      v at large v, e^v at very negative v, and softplus(v) - softplus(-v) = v.
Each of the conv oracle's test-only mistakes fails one of C1-C3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _torch_listing(x, w, b, silu):
    """The listing's nn.Conv1d(d, d, k, padding=k-1, groups=d) + cut + SiLU, fp64."""
    xt = torch.from_numpy(np.asarray(x, np.float64)).transpose(1, 2)  # (batch, D, L)
    D, W = w.shape
    conv = torch.nn.Conv1d(D, D, W, padding=W - 1, groups=D, bias=b is not None, dtype=torch.float64)
    with torch.no_grad():
        conv.weight.copy_(torch.from_numpy(np.asarray(w, np.float64))[:, None, :])
        if b is not None:
            conv.bias.copy_(torch.from_numpy(np.asarray(b, np.float64)))
        out = conv(xt)[:, :, :x.shape[1]]
        if silu:
            out = torch.nn.functional.silu(out)
    return out.transpose(1, 2).numpy()


CASES = [  # (batch, L, D, W, io, bias, silu)
    (2, 50, 7, 4, "f32", True, True),
    (1, 3, 5, 4, "f32", True, True),      # L < W
    (3, 33, 16, 1, "f32", False, True),   # width 1: pointwise
    (2, 40, 9, 3, "bf16", True, False),
    (1, 64, 12, 8, "bf16", False, True),
]


def _case(batch, L, D, W, io, bias, seed):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((batch, L, D)).astype(np.float32)
    x = np.array([synth.f32_to_bf16_bits(float(v)) for v in xf.ravel()], np.uint16).reshape(xf.shape) \
        if io == "bf16" else xf
    w = rng.standard_normal((D, W)).astype(np.float32) * 0.5
    b = rng.standard_normal(D).astype(np.float32) if bias else None
    return x, synth.to_f64(x, io), w, b


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_d%d_w%d_%s_bias%d_silu%d" % c)
def test_c1_listing_definition(case):
    batch, L, D, W, io, bias, silu = case
    x, x64, w, b = _case(batch, L, D, W, io, bias, 1)
    got = oracle.causal_conv1d(x, w, io, b, silu=silu)
    ref = _torch_listing(x64, w, b, silu)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_c2_numpy_convolve():
    x, x64, w, b = _case(2, 37, 6, 4, "f32", True, 2)
    got = oracle.causal_conv1d(x, w, "f32", b, silu=False)
    for bb in range(2):
        for d in range(6):
            ref = np.convolve(x64[bb, :, d], w[d, ::-1].astype(np.float64))[:37] + b[d]
            np.testing.assert_allclose(got[bb, :, d], ref, rtol=1e-12, atol=1e-12)


def test_c3_impulse_and_causality():
    W, L, D, t0 = 4, 20, 3, 7
    w = np.arange(1, D * W + 1, dtype=np.float32).reshape(D, W)
    x = np.zeros((1, L, D), np.float32)
    x[0, t0, :] = 1.0
    got = oracle.causal_conv1d(x, w, "f32", None, silu=False)[0]
    for d in range(D):
        want = np.zeros(L)
        for t in range(t0, t0 + W):
            want[t] = w[d, W - 1 - (t - t0)]   # newest input meets the last tap
        np.testing.assert_array_equal(got[:, d], want)
    # a change at step t1 leaves every earlier output unchanged
    rng = np.random.default_rng(3)
    xr = rng.standard_normal((1, L, D)).astype(np.float32)
    a = oracle.causal_conv1d(xr, w, "f32", None)
    xr[0, 12:] += 1.0
    b = oracle.causal_conv1d(xr, w, "f32", None)
    np.testing.assert_array_equal(a[0, :12], b[0, :12])
    assert np.all(a[0, 12] != b[0, 12])


def _pins_pass(mutation):
    try:
        for case in CASES[:2]:
            batch, L, D, W, io, bias, silu = case
            x, x64, w, b = _case(batch, L, D, W, io, bias, 1)
            got = oracle.causal_conv1d(x, w, io, b, silu=silu, mutation=mutation)
            np.testing.assert_allclose(got, _torch_listing(x64, w, b, silu), rtol=1e-12, atol=1e-12)
        return True
    except AssertionError:
        return False


def test_conv_pins_pass_unmutated():
    assert _pins_pass(0)


@pytest.mark.parametrize("mutation", sorted(oracle.CONV_MUTATIONS))
def test_conv_mutation_caught(mutation):
    assert not _pins_pass(mutation), oracle.CONV_MUTATIONS[mutation]


def _softplus_via_scan(v, bias=0.0):
    """y of a one-step scan with N = 1, A = 0, B = C = x = 1: exactly delta."""
    inp = {"x": np.ones((1, 1, 1), np.float32), "delta": np.full((1, 1, 1), v, np.float32),
           "A": np.zeros((1, 1), np.float32), "B": np.ones((1, 1, 1), np.float32),
           "C": np.ones((1, 1, 1), np.float32)}
    y, _ = oracle.selective_scan(inp, "f32", delta_softplus=True, delta_bias=np.full(1, bias, np.float32))
    return y[0, 0, 0]


def test_s1_softplus_values():
    assert _softplus_via_scan(0.0) == pytest.approx(np.log(2.0), rel=1e-15)
    assert _softplus_via_scan(1.5, bias=-1.5) == pytest.approx(np.log(2.0), rel=1e-15)   # the bias is added first
    assert _softplus_via_scan(40.0) == pytest.approx(40.0, rel=1e-15)
    assert _softplus_via_scan(-40.0) == pytest.approx(np.exp(-40.0), rel=1e-12)
    for v in (0.25, 1.0, 3.0, 7.5):
        assert _softplus_via_scan(v) - _softplus_via_scan(-v) == pytest.approx(v, rel=1e-14)
    # a plain scan without the flag takes delta as given
    inp = {"x": np.ones((1, 1, 1), np.float32), "delta": np.full((1, 1, 1), -3.0, np.float32),
           "A": np.zeros((1, 1), np.float32), "B": np.ones((1, 1, 1), np.float32),
           "C": np.ones((1, 1, 1), np.float32)}
    assert oracle.selective_scan(inp, "f32")[0][0, 0, 0] == -3.0
