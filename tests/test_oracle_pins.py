"""Pins of the fp64 oracle to things other than itself.

Each pin is a closed form, an invariant, a special case or brute force written
here independently of ``oracle/ssm_oracle.c``.  The pages print no worked
numeric example, so no value is copied from them.  ``test_mutation_caught``
plants each of the oracle's test-only mistakes and shows a pin fails.

Pins (pages are cited by title and section):
  P1  LTI convolution: with delta, B, C constant the recurrence equals
      convolution with Kbar = (C Bbar, C Abar Bbar, ...)  -- tildalice.io
      "Mamba 논문 리뷰", SSM의 이중 연산 모드.
  P2  Brute-force semiseparable form y = M x, M_ts = C_t^T (prod_{r=s+1}^t Abar_r) Bbar_s
      -- obsidian-dorae222 "Mamba-2", 1-세미분리 행렬.   P2b: rank of lower
      submatrices of M is <= N (same section).
  P3  ZOH is the exact solution of h' = a h + B x for inputs held over each
      step (yongggg.tistory.com review, 연속 신호에서 이산 신호로; tildalice.io
      이산화): closed form for constant inputs, and RK4 integration of the ODE.
  P4  Limits of delta (tildalice.io, Δ의 직관적 이해): large delta forgets the
      state and takes the input (h -> -B x / a); small delta keeps the state.
  P5  ZOH and the simplified Bbar = delta B differ by O(delta^2).
  P6  Degenerate cases: B = 0 or C = 0 leaves D x silu(z); N = 1, A = 0 is a
      prefix sum of delta B x.
  P7  Chaining through h0 / h_last.
  P8  SSD: the chunked algorithm equals the expanded recurrence for every chunk
      size, and the per-head brute-force M.
  P9  Associativity: a tree-order parallel prefix over (Abar, Bbar x) pairs
      equals the sequential fold (tildalice.io, 병렬 스캔).
  P10 Linearity in x.   P11 Causality.
"""
import numpy as np
import pytest

import oracle


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _f32(a):
    return np.asarray(a, np.float32)


def _inputs(rng, batch, L, D, N, z=True, Dk=True, a_lo=-2.0, a_hi=-0.2, d_lo=0.01, d_hi=0.6):
    inp = {
        "x": _f32(rng.standard_normal((batch, L, D))),
        "delta": _f32(rng.uniform(d_lo, d_hi, (batch, L, D))),
        "A": _f32(rng.uniform(a_lo, a_hi, (D, N))),
        "B": _f32(rng.standard_normal((batch, L, N))),
        "C": _f32(rng.standard_normal((batch, L, N))),
    }
    if Dk:
        inp["D"] = _f32(rng.standard_normal(D))
    if z:
        inp["z"] = _f32(rng.standard_normal((batch, L, D)))
    return inp


def _discretise(delta, a, B, euler):
    """Abar, Bbar for one step (fp64): Abar = exp(delta a), ZOH Bbar = (exp(delta a) - 1)/a B."""
    Abar = np.exp(delta * a)
    if euler:
        return Abar, delta * B
    return Abar, np.where(a != 0, np.expm1(delta * a) / np.where(a == 0, 1.0, a), delta) * B


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


# ----------------------------------------------------------------------------- P1
def pin_lti_convolution(mutation=0, euler=False):
    rng = np.random.default_rng(11)
    batch, L, D, N = 1, 40, 3, 4
    inp = _inputs(rng, batch, L, D, N, z=False, Dk=False)
    dconst = _f32(rng.uniform(0.05, 0.5, D))
    inp["delta"] = np.broadcast_to(dconst, (batch, L, D)).copy()
    Bc, Cc = _f32(rng.standard_normal(N)), _f32(rng.standard_normal(N))
    inp["B"] = np.broadcast_to(Bc, (batch, L, N)).copy()
    inp["C"] = np.broadcast_to(Cc, (batch, L, N)).copy()
    y, _ = oracle.selective_scan(inp, "f32", euler=euler, mutation=mutation)
    x = inp["x"].astype(np.float64)
    for d in range(D):
        a = inp["A"][d].astype(np.float64)
        Abar, Bbar = _discretise(float(dconst[d]), a, Bc.astype(np.float64), euler)
        K = np.array([np.sum(Cc.astype(np.float64) * Abar ** k * Bbar) for k in range(L)])
        ref = np.convolve(x[0, :, d], K)[:L]
        if _rel(y[0, :, d], ref) > 1e-12:
            return False
    return True


# ----------------------------------------------------------------------------- P2
def _brute_M(delta, A_row, B, C, euler):
    """M[t, s] = sum_n C[t,n] prod_{r=s+1}^{t} Abar[r,n] Bbar[s,n], s <= t."""
    L, N = B.shape
    Abar = np.exp(delta[:, None] * A_row[None, :])
    Bbar = np.stack([_discretise(delta[s], A_row, B[s], euler)[1] for s in range(L)])
    M = np.zeros((L, L))
    for t in range(L):
        for s in range(t + 1):
            prod = np.ones(N)
            for r in range(s + 1, t + 1):
                prod = prod * Abar[r]
            M[t, s] = np.sum(C[t] * prod * Bbar[s])
    return M


def pin_brute_force(mutation=0, euler=False, z=True):
    rng = np.random.default_rng(12)
    batch, L, D, N = 2, 11, 3, 4
    inp = _inputs(rng, batch, L, D, N, z=z, Dk=True)
    y, _ = oracle.selective_scan(inp, "f32", euler=euler, mutation=mutation)
    f = {k: v.astype(np.float64) for k, v in inp.items()}
    for b in range(batch):
        for d in range(D):
            M = _brute_M(f["delta"][b, :, d], f["A"][d], f["B"][b], f["C"][b], euler)
            ref = M @ f["x"][b, :, d] + f["D"][d] * f["x"][b, :, d]
            if z:
                ref = ref * _silu(f["z"][b, :, d])
            if _rel(y[b, :, d], ref) > 1e-12:
                return False
    return True


def test_p2b_semiseparable_rank():
    """Every submatrix of M inside the lower triangle has rank <= N."""
    rng = np.random.default_rng(13)
    L, N = 14, 3
    delta = rng.uniform(0.05, 0.7, L)
    A_row = rng.uniform(-2, -0.3, N)
    B, C = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    M = _brute_M(delta, A_row, B, C, euler=False)
    assert np.allclose(np.triu(M, 1), 0)
    ranks = set()
    for i in range(L):
        for j in range(1, i + 2):
            sub = M[i:, :j]  # rows t >= i, cols s < j <= i + 1: all s <= t
            sv = np.linalg.svd(sub, compute_uv=False)
            r = int(np.sum(sv > 1e-10 * sv[0])) if sv[0] > 0 else 0
            assert r <= N
            ranks.add(r)
    assert N in ranks  # the bound is reached: the construction is not degenerate


# ----------------------------------------------------------------------------- P3
def pin_closed_form(mutation=0):
    L = 30
    a, dl = np.float32(-0.7), np.float32(0.3)
    ones = np.ones((1, L, 1), np.float32)
    inp = {"x": ones, "delta": ones * dl, "A": np.full((1, 1), a, np.float32), "B": ones.copy(), "C": ones.copy()}
    t = np.arange(L)
    a64, d64 = float(a), float(dl)
    y, _ = oracle.selective_scan(inp, "f32", mutation=mutation)
    zoh = (np.exp(a64 * d64 * (t + 1)) - 1.0) / a64
    ok = _rel(y[0, :, 0], zoh) < 1e-13
    y, _ = oracle.selective_scan(inp, "f32", euler=True, mutation=mutation)
    eul = d64 * (1.0 - np.exp(a64 * d64 * (t + 1))) / (1.0 - np.exp(a64 * d64))
    return ok and _rel(y[0, :, 0], eul) < 1e-13


def _rk4_ode(a, forcing, h, T, steps):
    """Integrate h' = a*h + forcing on [0, T] with classic RK4 (elementwise)."""
    dt = T / steps
    for _ in range(steps):
        k1 = a * h + forcing
        k2 = a * (h + 0.5 * dt * k1) + forcing
        k3 = a * (h + 0.5 * dt * k2) + forcing
        k4 = a * (h + dt * k3) + forcing
        h = h + dt / 6.0 * (k1 + 2 * k2 + 2 * k3 + k4)
    return h


def pin_ode_zoh(mutation=0):
    """ZOH Bbar makes the recurrence the exact ODE solution with inputs held per step."""
    rng = np.random.default_rng(14)
    L, N = 8, 3
    inp = _inputs(rng, 1, L, 1, N, z=False, Dk=False, d_lo=0.05, d_hi=0.8)
    y, hl = oracle.selective_scan(inp, "f32", mutation=mutation)
    f = {k: v.astype(np.float64) for k, v in inp.items()}
    a = f["A"][0]
    h = np.zeros(N)
    for t in range(L):
        h = _rk4_ode(a, f["B"][0, t] * f["x"][0, t, 0], h, f["delta"][0, t, 0], 2000)
        if abs(y[0, t, 0] - np.sum(f["C"][0, t] * h)) > 1e-11 * (1 + abs(y[0, t, 0])):
            return False
    return _rel(hl[0, 0], h) < 1e-11


# ----------------------------------------------------------------------------- P4
def pin_limits(mutation=0):
    rng = np.random.default_rng(15)
    L, D, N = 12, 2, 4
    inp = _inputs(rng, 1, L, D, N, z=False, Dk=False, a_lo=-3.0, a_hi=-0.5)
    # large delta: Abar ~ 0, h_t = -B_t x_t / a exactly in the limit
    inp["delta"] = np.full((1, L, D), 200.0, np.float32)
    y, _ = oracle.selective_scan(inp, "f32", mutation=mutation)
    f = {k: v.astype(np.float64) for k, v in inp.items()}
    for d in range(D):
        h = -f["B"][0] * f["x"][0, :, d:d + 1] / f["A"][d][None, :]
        if _rel(y[0, :, d], np.sum(f["C"][0] * h, axis=1)) > 1e-12:
            return False
    # tiny delta: the state is kept and the input ignored
    inp["delta"] = np.full((1, L, D), 1e-9, np.float32)
    h0 = rng.standard_normal((1, D, N))
    y, hl = oracle.selective_scan(inp, "f32", h0=h0, mutation=mutation)
    for d in range(D):
        if _rel(y[0, :, d], f["C"][0] @ h0[0, d]) > 1e-7:
            return False
    return _rel(hl, h0) < 1e-7


# ----------------------------------------------------------------------------- P5
def test_p5_zoh_to_euler():
    """One step from h = 0: (ZOH - Euler) / (delta^2 a B x / 2) -> 1 as delta -> 0."""
    for eps in (1e-2, 1e-3):
        inp = {"x": np.full((1, 1, 1), 0.75, np.float32), "delta": np.full((1, 1, 1), eps, np.float32),
               "A": np.full((1, 1), -1.5, np.float32), "B": np.full((1, 1, 1), 1.25, np.float32),
               "C": np.ones((1, 1, 1), np.float32)}
        yz, _ = oracle.selective_scan(inp, "f32")
        ye, _ = oracle.selective_scan(inp, "f32", euler=True)
        d = float(np.float32(eps))
        ratio = (yz[0, 0, 0] - ye[0, 0, 0]) / (d * d * -1.5 * 1.25 * 0.75 / 2)
        assert abs(ratio - 1) < 2 * d


# ----------------------------------------------------------------------------- P6
def pin_degenerate(mutation=0):
    rng = np.random.default_rng(16)
    L, D, N = 20, 3, 4
    ok = True
    for zero in ("B", "C"):
        inp = _inputs(rng, 1, L, D, N, z=True, Dk=True)
        inp[zero] = np.zeros_like(inp[zero])
        y, _ = oracle.selective_scan(inp, "f32", mutation=mutation)
        f = {k: v.astype(np.float64) for k, v in inp.items()}
        ref = f["D"][None, :] * f["x"][0] * _silu(f["z"][0])
        ok = ok and _rel(y[0], ref) < 1e-14
    # N = 1, A = 0: h_t = sum_{s<=t} delta_s B_s x_s
    inp = _inputs(rng, 1, L, 1, 1, z=False, Dk=False)
    inp["A"] = np.zeros((1, 1), np.float32)
    y, _ = oracle.selective_scan(inp, "f32", mutation=mutation)
    f = {k: v.astype(np.float64) for k, v in inp.items()}
    h = np.cumsum(f["delta"][0, :, 0] * f["B"][0, :, 0] * f["x"][0, :, 0])
    return ok and _rel(y[0, :, 0], f["C"][0, :, 0] * h) < 1e-12


# ----------------------------------------------------------------------------- P7
def test_p7_chaining():
    rng = np.random.default_rng(17)
    L, D, N = 50, 3, 5
    inp = _inputs(rng, 2, L, D, N)
    y, hl = oracle.selective_scan(inp, "f32")
    for L1 in (1, 17, 32, 49):
        a = {k: (v[:, :L1] if v.ndim == 3 else v) for k, v in inp.items()}
        b = {k: (v[:, L1:] if v.ndim == 3 else v) for k, v in inp.items()}
        ya, ha = oracle.selective_scan(a, "f32")
        yb, hb = oracle.selective_scan(b, "f32", h0=ha)
        assert np.array_equal(np.concatenate([ya, yb], axis=1), y)
        assert np.array_equal(hb, hl)


# ----------------------------------------------------------------------------- P8
def _ssd_inputs(rng, batch, L, H, P, N, G):
    return {"x": _f32(rng.standard_normal((batch, L, H, P))),
            "delta": _f32(rng.uniform(0.01, 0.5, (batch, L, H))),
            "A": _f32(-np.exp(rng.uniform(0, 2.0, H))),
            "B": _f32(rng.standard_normal((batch, L, G, N))),
            "C": _f32(rng.standard_normal((batch, L, G, N))),
            "D": _f32(rng.standard_normal(H))}


@pytest.mark.parametrize("euler", [False, True])
def test_p8_ssd_chunk_size_invariance(euler):
    rng = np.random.default_rng(18)
    batch, L, H, P, N, G = 2, 67, 4, 3, 5, 2
    inp = _ssd_inputs(rng, batch, L, H, P, N, G)
    h0 = rng.standard_normal((batch, H, P, N))
    y, hl = oracle.ssd(inp, "f32", ngroups=G, euler=euler, h0=h0)
    for q in (1, 2, 16, 64, L):
        r = oracle.ssd_chunked(inp, "f32", q, ngroups=G, euler=euler, h0=h0)
        assert _rel(r["y"], y) < 1e-12, q
        assert _rel(r["h_last"], hl) < 1e-12, q


def test_p8_ssd_brute_force():
    """SSD per head equals y = M x with the head's scalar decay (Q = L is pure L o CB^T)."""
    rng = np.random.default_rng(19)
    batch, L, H, P, N, G = 1, 9, 2, 2, 3, 1
    inp = _ssd_inputs(rng, batch, L, H, P, N, G)
    y, _ = oracle.ssd(inp, "f32")
    f = {k: v.astype(np.float64) for k, v in inp.items()}
    for h in range(H):
        M = _brute_M(f["delta"][0, :, h], np.full(N, f["A"][h]), f["B"][0, :, 0], f["C"][0, :, 0], False)
        for p in range(P):
            ref = M @ f["x"][0, :, h, p] + f["D"][h] * f["x"][0, :, h, p]
            assert _rel(y[0, :, h, p], ref) < 1e-12
    r = oracle.ssd_chunked(inp, "f32", L)
    assert _rel(r["y"], y) < 1e-12


def test_ssd_equals_scan_with_expanded_inputs():
    """The SSD entry maps (h, p) -> channel, head delta/A -> every p, group B/C -> its heads."""
    rng = np.random.default_rng(20)
    batch, L, H, P, N, G = 2, 13, 4, 2, 3, 2
    inp = _ssd_inputs(rng, batch, L, H, P, N, G)
    y, _ = oracle.ssd(inp, "f32", ngroups=G)
    for h in range(H):
        g = h // (H // G)
        s = {"x": inp["x"][:, :, h, :], "delta": np.repeat(inp["delta"][:, :, h:h + 1], P, axis=2),
             "A": np.full((P, N), inp["A"][h], np.float32), "B": inp["B"][:, :, g], "C": inp["C"][:, :, g],
             "D": np.full(P, inp["D"][h], np.float32)}
        ys, _ = oracle.selective_scan(s, "f32")
        assert _rel(y[:, :, h, :], ys) < 1e-14


# ----------------------------------------------------------------------------- P9
def test_p9_tree_order_scan():
    """Hillis-Steele inclusive scan with (a1,b1) o (a2,b2) = (a1 a2, a2 b1 + b2)."""
    rng = np.random.default_rng(21)
    L, D, N = 37, 2, 3
    inp = _inputs(rng, 1, L, D, N, z=False, Dk=False)
    y, hl = oracle.selective_scan(inp, "f32")
    f = {k: v.astype(np.float64) for k, v in inp.items()}
    for d in range(D):
        a, b = [], []
        for t in range(L):
            Ab, Bb = _discretise(f["delta"][0, t, d], f["A"][d], f["B"][0, t], False)
            a.append(Ab)
            b.append(Bb * f["x"][0, t, d])
        a, b = np.array(a), np.array(b)
        k = 1
        while k < L:
            a2, b2 = a.copy(), b.copy()
            a2[k:] = a[:-k] * a[k:]
            b2[k:] = a[k:] * b[:-k] + b[k:]
            a, b = a2, b2
            k *= 2
        assert _rel(y[0, :, d], np.sum(f["C"][0] * b, axis=1)) < 1e-13
        assert _rel(hl[0, d], b[-1]) < 1e-13


# ----------------------------------------------------------------------------- P10/P11
def test_p10_linearity():
    rng = np.random.default_rng(22)
    L, D, N = 25, 3, 4
    inp = _inputs(rng, 1, L, D, N, z=False, Dk=True)
    x1 = _f32(np.round(rng.standard_normal((1, L, D)) * 256) / 256)
    x2 = _f32(np.round(rng.standard_normal((1, L, D)) * 256) / 256)
    ys = []
    for x in (x1, x2, _f32(2 * x1 + x2)):
        ys.append(oracle.selective_scan(dict(inp, x=x), "f32")[0])
    assert _rel(ys[2], 2 * ys[0] + ys[1]) < 1e-13


def test_p11_causality():
    rng = np.random.default_rng(23)
    L, D, N = 30, 3, 4
    inp = _inputs(rng, 1, L, D, N)
    y, _ = oracle.selective_scan(inp, "f32")
    for t0 in (0, 7, 29):
        for key in ("x", "delta"):
            p = {k: v.copy() for k, v in inp.items()}
            p[key][0, t0] += 0.5
            yp, _ = oracle.selective_scan(p, "f32")
            assert np.array_equal(yp[:, :t0], y[:, :t0])
            assert not np.array_equal(yp[:, t0:], y[:, t0:])


# ----------------------------------------------------------------------------- wiring
PINS = {
    "P1_lti_zoh": lambda m: pin_lti_convolution(m, euler=False),
    "P1_lti_euler": lambda m: pin_lti_convolution(m, euler=True),
    "P2_brute_zoh": lambda m: pin_brute_force(m, euler=False, z=True),
    "P2_brute_euler": lambda m: pin_brute_force(m, euler=True, z=False),
    "P3_closed_form": pin_closed_form,
    "P3_ode": pin_ode_zoh,
    "P4_limits": pin_limits,
    "P6_degenerate": pin_degenerate,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    assert PINS[name](0), name


@pytest.mark.parametrize("mutation", sorted(oracle.MUTATIONS))
def test_mutation_caught(mutation):
    """A planted mistake in the oracle makes at least one pin fail."""
    failed = [n for n, f in PINS.items() if not f(mutation)]
    assert failed, "mutation %d (%s) passed every pin" % (mutation, oracle.MUTATIONS[mutation])
