"""fp64 CPU oracle for the selective scan (S6) and the SSD chunked form.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package; the GPU path never does,
and it shares no code with it.

* ``selective_scan`` / ``ssd`` run the plain recurrence in C (``ssm_oracle.c``),
  one independent row per thread task.  Discretisation per the tildalice.io
  review "Mamba 논문 리뷰" (section 이산화): Abar = exp(delta*A),
  Bbar = (delta*A)^-1 (exp(delta*A) - 1) delta*B; recurrence h_t = Abar h_{t-1}
  + Bbar x_t; readout y_t = C_t h_t, plus D x_t (yongggg.tistory.com review,
  State Space Model section) and the SiLU(z) gate (tildalice.io, Mamba block).
* ``ssd_chunked`` (numpy, fp64) takes the steps of the SSD tiling algorithm of
  the obsidian-dorae222 "Mamba-2" page (section SSD 타일링 알고리즘) in order --
  chunk cumulative decay, chunk states, state passing, chunk scan -- and returns
  every intermediate so that each GPU step can be checked on its own.  It is
  pinned to the recurrence by the tests (any chunk size gives the same y).
* ``selective_scan(..., delta_softplus=True, delta_bias=b)`` first replaces
  delta by softplus(delta + b) (tildalice.io SelectiveSSM listing: delta is
  the softplus of its projection, which carries a bias).
* ``selective_scan_bwd`` is the reverse-mode derivative of ``selective_scan``
  (the recomputation-based backward of tildalice.io 역전파 시 재계산 computes
  the same numbers): the forward states of each row, then the adjoint
  recurrence lam_t = C_t g_t + Abar_{t+1} lam_{t+1} backwards in time.
* ``ssd_bwd`` is the SSD's gradient as the scan's: each channel (h, p) runs
  the selective recurrence with tied per-head (delta, A, D) and per-group
  (B, C) parameters, so the scan backward of the untied channels, with the
  tied copies' gradients added, is its derivative.
* ``causal_conv1d`` is the Mamba block's per-channel Conv1D of width k with
  k - 1 steps of zero padding cut back to the first L outputs, then SiLU
  (tildalice.io, Mamba 블록 아키텍처 and the SelectiveSSM listing), as a direct
  sum in C.
* ``mamba_block`` composes one Mamba block in fp64 in the order of the block
  figure and listing of the same page: in_proj, conv + SiLU, x_proj (B, C,
  dt), dt_proj, the selective scan with softplus(delta + bias), the D skip and
  the SiLU(z) gate, out_proj.  Matrix products are numpy's; the conv and the
  scan are the functions above.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "libssm_oracle.so")

MUTATIONS = {
    1: "skip term D*x dropped",
    2: "sign of the exponent flipped",
    3: "B and C swapped",
    4: "x read one step late",
    5: "Euler Bbar used in place of ZOH",
    6: "readout uses the wrong state index",
    7: "gate sigmoid(z) in place of SiLU(z)",
}


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                               "-std=c11", _SRC, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_selective_scan.restype = ci
        lib.oracle_selective_scan.argtypes = [i64, i64, i64, i64, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                              vp, vp, ci, ci, ci, vp]
        lib.oracle_selective_scan_bwd.restype = ci
        lib.oracle_selective_scan_bwd.argtypes = [i64, i64, i64, i64, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp, ci, vp, vp,
                                                  ci, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci]
        lib.oracle_causal_conv1d.restype = ci
        lib.oracle_causal_conv1d.argtypes = [i64, i64, i64, i64, ci, vp, vp, vp, ci, vp, ci]
        lib.oracle_ssd.restype = ci
        lib.oracle_ssd.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp,
                                   vp, ci, ci]
        _lib = lib
    return _lib


def threads() -> int:
    """Host threads the oracle uses: every core in this process's affinity mask."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _io(a, io):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype={"bf16": np.uint16, "f32": np.float32, "f64": np.float64}[io])


def _mode(io):
    return {"f32": 0, "bf16": 1, "f64": 2}[io]


def selective_scan(inp: dict, io: str, euler: bool = False, h0=None, rows=None, nthreads=None, mutation=0,
                   delta_softplus: bool = False, delta_bias=None):
    """Reference scan.

    inp: x, delta (batch, L, D); A (D, N) fp32; B, C (batch, L, N); optional
    D (D,) fp32 and z (batch, L, D).  bf16 tensors are uint16 bit patterns.
    h0: optional (batch, D, N).  rows: optional flat ids b*D + d.
    delta_softplus: delta <- softplus(delta + delta_bias) (delta_bias (D,)
    fp32, optional).
    Returns (y, h_last): (batch, L, D) and (batch, D, N) float64, or
    (nrows, L) and (nrows, N) when rows is given.
    """
    x, dl, B, C, z = (_io(inp.get(k), io) for k in ("x", "delta", "B", "C", "z"))
    A, Dk = _c(inp["A"], np.float32), _c(inp.get("D"), np.float32)
    batch, L, D = x.shape
    N = A.shape[1]
    assert dl.shape == x.shape and B.shape == (batch, L, N) and C.shape == (batch, L, N) and A.shape == (D, N)
    h0c = _c(h0, np.float64)
    if h0c is not None:
        assert h0c.shape == (batch, D, N)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = batch * D if r is None else len(r)
    y = np.empty((nr, L), np.float64)
    hl = np.empty((nr, N), np.float64)
    rc = _load().oracle_selective_scan(batch, L, D, N, _mode(io), 1 if euler else 0, _ptr(x),
                                       _ptr(dl), _ptr(A), _ptr(B), _ptr(C), _ptr(Dk), _ptr(z), _ptr(h0c), _ptr(r),
                                       nr, _ptr(y), _ptr(hl), nthreads or threads(), mutation,
                                       1 if delta_softplus else 0, _ptr(_c(delta_bias, np.float32)))
    if rc != 0:
        raise ValueError("oracle_selective_scan rejected its arguments")
    if r is None:
        return y.reshape(batch, D, L).transpose(0, 2, 1).copy(), hl.reshape(batch, D, N)
    return y, hl


def ssd(inp: dict, io: str, ngroups: int = 1, euler: bool = False, h0=None, rows=None, nthreads=None,
        mutation=0):
    """Reference SSD as the expanded scan.

    inp: x (batch, L, H, P); delta (batch, L, H); A (H,) fp32; B, C
    (batch, L, G, N); optional D (H,) fp32.  h0: optional (batch, H, P, N).
    rows: optional flat ids b*H*P + h*P + p.
    Returns (y, h_last): (batch, L, H, P) and (batch, H, P, N), or row-major
    (nrows, L) and (nrows, N) when rows is given.
    """
    x, dl, B, C = (_io(inp.get(k), io) for k in ("x", "delta", "B", "C"))
    A, Dk = _c(inp["A"], np.float32), _c(inp.get("D"), np.float32)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert G == ngroups and dl.shape == (batch, L, H) and A.shape == (H,) and C.shape == B.shape
    h0c = _c(h0, np.float64)
    if h0c is not None:
        assert h0c.shape == (batch, H, P, N)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = batch * H * P if r is None else len(r)
    y = np.empty((nr, L), np.float64)
    hl = np.empty((nr, N), np.float64)
    rc = _load().oracle_ssd(batch, L, H, P, N, G, _mode(io), 1 if euler else 0, _ptr(x), _ptr(dl),
                            _ptr(A), _ptr(B), _ptr(C), _ptr(Dk), _ptr(h0c), _ptr(r), nr, _ptr(y), _ptr(hl),
                            nthreads or threads(), mutation)
    if rc != 0:
        raise ValueError("oracle_ssd rejected its arguments")
    if r is None:
        return (y.reshape(batch, H, P, L).transpose(0, 3, 1, 2).copy(), hl.reshape(batch, H, P, N))
    return y, hl


BWD_MUTATIONS = {1: "adjoint carried without the decay Abar"}


def selective_scan_bwd(inp: dict, io: str, dy, dy_io: str = None, euler: bool = False, h0=None,
                       delta_softplus: bool = False, delta_bias=None, mutation: int = 0, nthreads=None) -> dict:
    """Gradients of sum(dy * y) for y = selective_scan(inp, ...), fp64.

    Same inputs as selective_scan; dy (batch, L, D) in dy_io (default io).
    Returns dict: dx, ddelta (delta as passed in), dz (if z), dA, dB, dC, dD (if
    D), ddelta_bias (if delta_softplus and delta_bias), dh0 (if h0).
    """
    x, dl, B, C, z = (_io(inp.get(k), io) for k in ("x", "delta", "B", "C", "z"))
    A, Dk = _c(inp["A"], np.float32), _c(inp.get("D"), np.float32)
    batch, L, D = x.shape
    N = A.shape[1]
    dyi = _io(dy, dy_io or io)
    h0c = _c(h0, np.float64)
    dbi = _c(delta_bias, np.float32)
    out = {k: np.empty((batch, L, D)) for k in ("dx", "ddelta")}
    out["dA"] = np.empty((D, N))
    out["dB"], out["dC"] = np.empty((batch, L, N)), np.empty((batch, L, N))
    if z is not None:
        out["dz"] = np.empty((batch, L, D))
    if Dk is not None:
        out["dD"] = np.empty(D)
    if delta_softplus and dbi is not None:
        out["ddelta_bias"] = np.empty(D)
    if h0c is not None:
        out["dh0"] = np.empty((batch, D, N))
    rc = _load().oracle_selective_scan_bwd(batch, L, D, N, _mode(io), 1 if euler else 0, _ptr(x), _ptr(dl), _ptr(A),
                                           _ptr(B), _ptr(C), _ptr(Dk), _ptr(z), _ptr(h0c), 1 if delta_softplus else 0,
                                           _ptr(dbi), _ptr(dyi), _mode(dy_io or io), _ptr(out["dx"]),
                                           _ptr(out["ddelta"]), _ptr(out.get("dz")), _ptr(out["dA"]), _ptr(out["dB"]),
                                           _ptr(out["dC"]), _ptr(out.get("dD")), _ptr(out.get("ddelta_bias")),
                                           _ptr(out.get("dh0")), nthreads or threads(), mutation)
    if rc != 0:
        raise ValueError("oracle_selective_scan_bwd failed")
    return out


SSD_BWD_MUTATIONS = {1: "head h read from group h % G instead of h / (H / G)",
                     2: "ddelta taken from the head's first channel only"}


def ssd_bwd(inp: dict, io: str, dy, ngroups: int = 1, euler: bool = False, h0=None, dy_io: str = None,
            mutation: int = 0, nthreads=None) -> dict:
    """Gradients of sum(dy * y) for (y, _) = ssd(inp, ...), fp64.

    Every channel (h, p) of the SSD runs the selective recurrence with the
    head's scalar A, its delta and the B, C of its group (obsidian-dorae222
    "Mamba-2", SSM-Attention 동치성 and SSD 타일링 알고리즘: the chunked form
    computes that recurrence exactly).  So the SSD is the selective scan of
    its untied channels, and its gradient is selective_scan_bwd of those
    channels with the gradients of tied copies added: over p for delta and D,
    over p and n for A, over the heads of a group for B and C.
    inp as for ssd; dy (batch, L, H, P) in dy_io (default io).
    Returns dx (batch, L, H, P), ddelta (batch, L, H), dA (H,), dB, dC
    (batch, L, G, N), dD (H,) if D, dh0 (batch, H, P, N) if h0.
    """
    x, dl, B, C = (_f64(inp.get(k), io) for k in ("x", "delta", "B", "C"))
    A = np.asarray(inp["A"], np.float32)
    Dk = None if inp.get("D") is None else np.asarray(inp["D"], np.float32)
    dyf = _f64(dy, dy_io or io)
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert G == ngroups and H % G == 0 and dl.shape == (batch, L, H) and A.shape == (H,) and dyf.shape == x.shape
    hpg = H // G
    out = {"dx": np.zeros((batch, L, H, P)), "ddelta": np.zeros((batch, L, H)), "dA": np.zeros(H),
           "dB": np.zeros((batch, L, G, N)), "dC": np.zeros((batch, L, G, N))}
    if Dk is not None:
        out["dD"] = np.zeros(H)
    if h0 is not None:
        out["dh0"] = np.zeros((batch, H, P, N))
    for g in range(G):
        heads = np.arange(g * hpg, (g + 1) * hpg)
        src = heads % G if mutation == 1 else np.full(hpg, g)
        for k, h in enumerate(heads):
            # one head at a time: channels p of head h, B and C of its group
            sub = {"x": x[:, :, h, :], "delta": np.repeat(dl[:, :, h:h + 1], P, axis=2),
                   "A": np.full((P, N), A[h], np.float32), "B": B[:, :, src[k], :], "C": C[:, :, src[k], :]}
            if Dk is not None:
                sub["D"] = np.full(P, Dk[h], np.float32)
            h0h = None if h0 is None else np.asarray(h0, np.float64)[:, h]
            r = selective_scan_bwd(sub, "f64", dyf[:, :, h, :], euler=euler, h0=h0h, nthreads=nthreads)
            out["dx"][:, :, h, :] = r["dx"]
            out["ddelta"][:, :, h] = r["ddelta"][:, :, 0] if mutation == 2 else r["ddelta"].sum(axis=2)
            out["dA"][h] = r["dA"].sum()
            out["dB"][:, :, g, :] += r["dB"]
            out["dC"][:, :, g, :] += r["dC"]
            if Dk is not None:
                out["dD"][h] = r["dD"].sum()
            if h0 is not None:
                out["dh0"][:, h] = r["dh0"]
    return out


CONV_MUTATIONS = {1: "taps reversed", 2: "window one step late", 3: "sigmoid in place of SiLU"}


def causal_conv1d(x, weight, io: str, bias=None, silu: bool = True, mutation: int = 0):
    """Causal depthwise convolution (+ bias, + SiLU), fp64.

    x: (batch, L, D) in the io dtype (bf16 as uint16 bit patterns); weight
    (D, W) fp32; bias (D,) fp32 or None.  out[b,t,d] = bias[d] +
    sum_k weight[d,k] x[b, t-(W-1)+k, d] with x = 0 before t = 0, then SiLU.
    Returns (batch, L, D) float64.
    """
    xc = _io(x, io)
    w = _c(weight, np.float32)
    bc = _c(bias, np.float32)
    batch, L, D = xc.shape
    assert w.ndim == 2 and w.shape[0] == D and (bc is None or bc.shape == (D,))
    out = np.empty((batch, L, D), np.float64)
    rc = _load().oracle_causal_conv1d(batch, L, D, w.shape[1], _mode(io), _ptr(xc), _ptr(w),
                                      _ptr(bc), 1 if silu else 0, _ptr(out), mutation)
    if rc != 0:
        raise ValueError("oracle_causal_conv1d rejected its arguments")
    return out


def _f64(a, io):
    if a is None:
        return None
    if io == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if io == "f64":
        return np.asarray(a, np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


def ssd_chunked(inp: dict, io: str, chunk: int, ngroups: int = 1, euler: bool = False, h0=None):
    """The SSD tiling algorithm, fp64, with every intermediate.

    Steps (obsidian-dorae222 "Mamba-2", SSD 타일링 알고리즘; the inter-chunk
    term read as the decay-weighted sum over the chunk, the only reading under
    which the result equals the semiseparable form y = M x):
      1. a_t = delta_t * A_h; A_cum = inclusive cumulative sum of a inside each
         chunk; beta_t = expm1(a_t)/A_h (ZOH; delta_t if A_h = 0) or delta_t.
      2. chunk state: S_loc[c] = sum_j exp(A_cum_end - A_cum_j) beta_j x_j B_j^T
      3. state passing: S_in[0] = h0 or 0, S_in[c+1] = exp(A_cum_end[c]) S_in[c] + S_loc[c]
      4. chunk scan: y_i = sum_{j<=i in chunk} exp(A_cum_i - A_cum_j) (C_i . B_j) beta_j x_j
                          + exp(A_cum_i) S_in[c] C_i + D_h x_i
    The last chunk may be shorter than `chunk`.
    Returns dict with y (batch, L, H, P), A_cum (batch, H, L), beta (batch, H, L),
    S_loc (batch, nc, H, P, N), S_in (batch, nc, H, P, N), h_last (batch, H, P, N).
    """
    x = _f64(inp["x"], io)
    dl = _f64(inp["delta"], io)
    B = _f64(inp["B"], io)
    C = _f64(inp["C"], io)
    # A and D: fp32 parameters, or fp64 as given (io "f64")
    A = _f64(inp["A"], "f64" if io == "f64" else "f32")
    Dk = _f64(inp.get("D"), "f64" if io == "f64" else "f32")
    batch, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // ngroups
    gidx = np.arange(H) // hpg
    Bh = B[:, :, gidx, :]  # (batch, L, H, N)
    Ch = C[:, :, gidx, :]
    a = dl * A[None, None, :]  # (batch, L, H)
    if euler:
        beta = dl.copy()
    else:
        with np.errstate(divide="ignore", invalid="ignore"):
            beta = np.where(A[None, None, :] != 0, np.expm1(a) / np.where(A == 0, 1.0, A)[None, None, :], dl)
    nc = (L + chunk - 1) // chunk
    A_cum = np.empty((batch, L, H))
    for c in range(nc):
        s, e = c * chunk, min(L, (c + 1) * chunk)
        A_cum[:, s:e] = np.cumsum(a[:, s:e], axis=1)
    S_loc = np.zeros((batch, nc, H, P, N))
    S_in = np.zeros((batch, nc, H, P, N))
    y = np.zeros((batch, L, H, P))
    state = np.zeros((batch, H, P, N)) if h0 is None else np.asarray(h0, np.float64).copy()
    for c in range(nc):
        s, e = c * chunk, min(L, (c + 1) * chunk)
        Ac = A_cum[:, s:e]                      # (b, q, h)
        Aend = Ac[:, -1]                        # (b, h)
        w = np.exp(Aend[:, None, :] - Ac) * beta[:, s:e]          # (b, q, h)
        S_loc[:, c] = np.einsum("bqh,bqhp,bqhn->bhpn", w, x[:, s:e], Bh[:, s:e])
        S_in[:, c] = state
        state = np.exp(Aend)[:, :, None, None] * state + S_loc[:, c]
        # chunk scan
        q = e - s
        diff = Ac[:, :, None, :] - Ac[:, None, :, :]              # (b, i, j, h)
        causal = np.tril(np.ones((q, q), bool))[None, :, :, None]
        Lmask = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
        CB = np.einsum("bihn,bjhn->bijh", Ch[:, s:e], Bh[:, s:e])
        Wij = Lmask * CB * beta[:, None, s:e, :]                  # (b, i, j, h)
        y_intra = np.einsum("bijh,bjhp->bihp", Wij, x[:, s:e])
        y_inter = np.exp(Ac)[..., None] * np.einsum("bhpn,bihn->bihp", S_in[:, c], Ch[:, s:e])
        y[:, s:e] = y_intra + y_inter
        if Dk is not None:
            y[:, s:e] += Dk[None, None, :, None] * x[:, s:e]
    return {"y": y, "A_cum": A_cum.transpose(0, 2, 1).copy(), "beta": beta.transpose(0, 2, 1).copy(),
            "S_loc": S_loc, "S_in": S_in, "h_last": state}


BLOCK_MUTATIONS = {1: "x and z halves of in_proj swapped", 2: "B and C columns of x_proj swapped",
                   3: "dt_proj bias dropped", 4: "conv output without SiLU"}


def mamba_block(inp: dict, io: str, dstate: int, dt_rank: int, intermediates: bool = False, mutation: int = 0):
    """One Mamba block forward in fp64.

    inp (synth.block_inputs): u (batch, L, M); W_in (2E, M); conv_w (E, k),
    conv_b (E); W_x (>= 2N + R, E) with rows B | C | dt (any further rows are
    ignored); W_dt (E, R), b_dt (E); A (E, N); D (E); W_out (M, E).
    Steps (tildalice.io "Mamba 논문 리뷰", Mamba 블록 아키텍처 and the
    SelectiveSSM listing; delta is the softplus of dt_proj of the rank-R slice
    of x_proj, with dt_proj's bias):
        xz = u W_in^T;  x, z = xz[..., :E], xz[..., E:]
        xc = silu(conv(x) + conv_b)
        B, C, dt = split(xc W_x^T)
        delta_raw = dt W_dt^T
        y = scan(xc, softplus(delta_raw + b_dt), A, B, C) + D xc, times silu(z)
        out = y W_out^T
    Returns out (batch, L, M) float64 (and a dict of intermediates).
    """
    f = lambda k: _f64(inp[k], io)
    u, W_in, W_x, W_dt, W_out = f("u"), f("W_in"), f("W_x"), f("W_dt"), f("W_out")
    N, R = dstate, dt_rank
    E = W_in.shape[0] // 2
    xz = u @ W_in.T
    x, z = xz[..., :E], xz[..., E:]
    if mutation == 1:
        x, z = z, x
    xc = causal_conv1d(np.ascontiguousarray(x), inp["conv_w"], "f64", inp["conv_b"], silu=mutation != 4)
    xd = xc @ W_x.T
    Bm, Cm, dt = xd[..., :N], xd[..., N:2 * N], xd[..., 2 * N:2 * N + R]
    if mutation == 2:
        Bm, Cm = Cm, Bm
    draw = dt @ W_dt.T
    sc = {"x": xc, "delta": draw, "A": inp["A"], "B": np.ascontiguousarray(Bm), "C": np.ascontiguousarray(Cm),
          "D": inp["D"], "z": np.ascontiguousarray(z)}
    dbias = np.zeros_like(inp["b_dt"]) if mutation == 3 else inp["b_dt"]
    y, _ = selective_scan(sc, "f64", delta_softplus=True, delta_bias=dbias)
    out = y @ W_out.T
    if intermediates:
        return out, {"xz": xz, "xc": xc, "xd": xd, "delta_raw": draw, "y": y}
    return out
