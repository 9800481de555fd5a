"""Pins of the oracle's SSD backward (oracle.ssd_bwd).

S1  Central finite differences of the numpy chunked SSD forward
    (oracle.ssd_chunked, an implementation independent of the scan code the
    backward is built on) along random directions, for every input and
    h0: <grad, v> = (f(p + e v) - f(p - e v)) / 2e with f = sum(dy * y), with
    several chunks, two groups, zero-order hold and the simplified Bbar.
S2  Each planted mistake of oracle.SSD_BWD_MUTATIONS fails S1.
"""
import numpy as np
import pytest

import oracle


def _case(seed, batch=1, L=11, H=4, P=3, N=5, G=2, Dk=True, h0=True):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s)
    inp = {"x": f(batch, L, H, P), "delta": np.abs(f(batch, L, H)) * 0.4 + 0.05,
           "A": -np.exp(rng.uniform(-1, 1.5, H)), "B": f(batch, L, G, N), "C": f(batch, L, G, N)}
    if Dk:
        inp["D"] = f(H)
    # fp32-representable base point: the backward reads fp32 A and D
    inp = {k: np.asarray(v, np.float32).astype(np.float64) for k, v in inp.items()}
    hz = f(batch, H, P, N) if h0 else None
    dy = f(batch, L, H, P)
    return rng, inp, hz, dy


def _fd_check(grads, inp, hz, dy, G, euler, rng, chunk=4, eps=1e-5):
    def fval(i2, h2):
        y = oracle.ssd_chunked(i2, "f64", chunk=chunk, ngroups=G, euler=euler, h0=h2)["y"]
        return float((y * dy).sum())

    names = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD"}
    bad = []
    for k, gk in names.items():
        if k not in inp:
            continue
        v = rng.standard_normal(inp[k].shape)
        hi, lo = dict(inp), dict(inp)
        hi[k], lo[k] = inp[k] + eps * v, inp[k] - eps * v
        fd = (fval(hi, hz) - fval(lo, hz)) / (2 * eps)
        an = float((grads[gk] * v).sum())
        if not np.isclose(an, fd, rtol=1e-6, atol=1e-7):
            bad.append((k, an, fd))
    if hz is not None:
        v = rng.standard_normal(hz.shape)
        fd = (fval(inp, hz + eps * v) - fval(inp, hz - eps * v)) / (2 * eps)
        an = float((grads["dh0"] * v).sum())
        if not np.isclose(an, fd, rtol=1e-6, atol=1e-7):
            bad.append(("h0", an, fd))
    return bad


@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("h0", [False, True])
def test_ssd_bwd_finite_differences(euler, G, h0):
    rng, inp, hz, dy = _case(7 + G + 2 * h0, G=G, h0=h0)
    grads = oracle.ssd_bwd(inp, "f64", dy, ngroups=G, euler=euler, h0=hz, dy_io="f64")
    assert _fd_check(grads, inp, hz, dy, G, euler, rng) == []


def test_ssd_bwd_zero_A_head():
    # A_h = 0: beta -> delta, and dbeta/dA = delta^2 / 2 (the limit)
    rng, inp, hz, dy = _case(3, G=1, h0=True)
    inp["A"][1] = 0.0
    grads = oracle.ssd_bwd(inp, "f64", dy, ngroups=1, h0=hz, dy_io="f64")
    assert _fd_check(grads, inp, hz, dy, 1, False, rng) == []


@pytest.mark.parametrize("mutation", sorted(oracle.SSD_BWD_MUTATIONS))
def test_ssd_bwd_mutations_fail(mutation):
    rng, inp, hz, dy = _case(11, G=2, h0=True)
    grads = oracle.ssd_bwd(inp, "f64", dy, ngroups=2, h0=hz, dy_io="f64", mutation=mutation)
    assert _fd_check(grads, inp, hz, dy, 2, False, rng) != []
