"""Pins of the oracle's scan backward (oracle.selective_scan_bwd).

G1  torch float64 autograd of an independent torch implementation of the
    forward (a dense per-step loop over the (D, N) state written here from the
    discretisation of tildalice.io "Mamba 논문 리뷰", section 이산화, with the
    D skip and SiLU(z) gate), every gradient, several flag combinations.
G2  Central finite differences of the forward oracle (oracle.selective_scan)
    on random directions: <grad, v> = (f(p + e v) - f(p - e v)) / 2e with
    f = sum(dy * y).
The test-only mistake of the backward fails G1.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _inputs(rng, batch, L, D, N, z, Dk, zero_a=False):
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    inp = {"x": f(batch, L, D), "delta": np.abs(f(batch, L, D)) * 0.3 + 0.02,
           "A": -np.exp(rng.uniform(-1, 1, (D, N))).astype(np.float32), "B": f(batch, L, N), "C": f(batch, L, N)}
    if zero_a:
        inp["A"][0, :] = 0.0
        inp["A"][1, 1] = 0.0
    if Dk:
        inp["D"] = f(D)
    if z:
        inp["z"] = f(batch, L, D)
    return inp


def _torch_grads(inp, dy, euler, h0, softplus, dbias):
    T = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in inp.items()}
    h0t = None if h0 is None else torch.tensor(h0, requires_grad=True)
    dbt = None if dbias is None else torch.tensor(np.asarray(dbias, np.float64), requires_grad=True)
    x, dl, A, B, C = T["x"], T["delta"], T["A"], T["B"], T["C"]
    if softplus:
        dl = F.softplus(dl + (dbt if dbt is not None else 0.0))
    batch, L, D = x.shape
    N = A.shape[1]
    h = torch.zeros(batch, D, N, dtype=torch.float64) if h0t is None else h0t
    ys = []
    for t in range(L):
        u = dl[:, t, :, None] * A                     # (batch, D, N)
        if euler:
            c = dl[:, t, :, None].expand_as(u)
        else:
            # a = 0: the limit written as a series in u = delta a, so that its
            # derivative in a (delta^2 / 2) survives autograd
            safe = torch.where(A == 0, torch.ones_like(A), A)
            lim = dl[:, t, :, None] * (1 + u / 2 + u * u / 6)
            c = torch.where(A == 0, lim, torch.expm1(u) / safe)
        h = torch.exp(u) * h + c * B[:, t, None, :] * x[:, t, :, None]
        ys.append((h * C[:, t, None, :]).sum(-1))
    y = torch.stack(ys, 1)
    if "D" in T:
        y = y + T["D"] * x
    if "z" in T:
        y = y * F.silu(T["z"])
    (y * torch.from_numpy(dy)).sum().backward()
    g = {"d" + k: v.grad.numpy() for k, v in T.items()}
    if h0t is not None:
        g["dh0"] = h0t.grad.numpy()
    if dbt is not None:
        g["ddelta_bias"] = dbt.grad.numpy()
    return g


CASES = [  # (batch, L, D, N, z, D, euler, h0, softplus, bias, zero_a)
    (2, 17, 3, 4, True, True, False, True, False, False, False),
    (1, 23, 4, 3, False, False, False, False, False, False, True),
    (2, 11, 3, 5, True, True, True, True, False, False, False),
    (2, 19, 5, 4, True, True, False, True, True, True, False),
    (1, 9, 2, 2, False, True, False, False, True, False, False),
]


def _run(case, seed, mutation=0):
    batch, L, D, N, z, Dk, euler, h0, sp, bias, zero_a = case
    rng = np.random.default_rng(seed)
    inp = _inputs(rng, batch, L, D, N, z, Dk, zero_a)
    if sp:
        inp["delta"] = rng.standard_normal((batch, L, D)).astype(np.float32)
    dy = rng.standard_normal((batch, L, D))
    h0v = rng.standard_normal((batch, D, N)) if h0 else None
    dbias = (rng.standard_normal(D).astype(np.float32) - 2.0) if bias else None
    got = oracle.selective_scan_bwd(inp, "f32", dy, "f64", euler=euler, h0=h0v, delta_softplus=sp, delta_bias=dbias,
                                    mutation=mutation)
    return inp, dy, h0v, dbias, got


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_d%d_n%d_z%d_D%d_e%d_h%d_sp%d_bias%d_za%d" % c)
def test_g1_autograd(case):
    inp, dy, h0v, dbias, got = _run(case, 1)
    ref = _torch_grads(inp, dy, case[6], h0v, case[8], dbias)
    keys = {"dx", "ddelta", "dA", "dB", "dC"} | ({"dz"} if case[4] else set()) | ({"dD"} if case[5] else set()) | \
        ({"dh0"} if case[7] else set()) | ({"ddelta_bias"} if case[9] else set())
    assert keys == set(got), (keys, set(got))
    for k in keys:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-9, atol=1e-10, err_msg=k)


def test_bwd_mutation_caught():
    case = CASES[0]
    inp, dy, h0v, dbias, got = _run(case, 1, mutation=1)
    ref = _torch_grads(inp, dy, case[6], h0v, case[8], dbias)
    assert not np.allclose(got["dx"], ref["dx"], rtol=1e-9, atol=1e-10)


def test_g2_finite_differences():
    """Directional derivatives of f = sum(dy * y) along random directions in
    x, delta, A, B, C, D, z, h0 against the backward's gradients."""
    rng = np.random.default_rng(7)
    batch, L, D, N = 2, 15, 3, 4
    inp = _inputs(rng, batch, L, D, N, True, True)
    inp64 = {k: v.astype(np.float64) for k, v in inp.items()}
    dy = rng.standard_normal((batch, L, D))
    h0 = rng.standard_normal((batch, D, N))
    g = oracle.selective_scan_bwd(inp, "f32", dy, "f64", h0=h0)

    def f(p, hh):
        # A and D are float32 arguments of the oracle and cannot take fp64
        # perturbations; their gradients are covered by G1
        y, _ = oracle.selective_scan(p, "f64", h0=hh)
        return float((y * dy).sum())

    eps = 1e-6
    for k in ("x", "delta", "B", "C", "z"):
        v = rng.standard_normal(inp64[k].shape)
        pp = dict(inp64); pp[k] = inp64[k] + eps * v
        pm = dict(inp64); pm[k] = inp64[k] - eps * v
        fd = (f(pp, h0) - f(pm, h0)) / (2 * eps)
        an = float((g["d" + k] * v).sum())
        assert fd == pytest.approx(an, rel=1e-6, abs=1e-8), k
    v = rng.standard_normal(h0.shape)
    fd = (f(inp64, h0 + eps * v) - f(inp64, h0 - eps * v)) / (2 * eps)
    assert fd == pytest.approx(float((g["dh0"] * v).sum()), rel=1e-6, abs=1e-8)
