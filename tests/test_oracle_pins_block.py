"""Pin of the oracle's Mamba block composition (oracle.mamba_block).

B1: an independent float64 numpy evaluation of the block in matrix form,
derived from the equations rather than from any listing.  The pages' block
(tildalice.io "Mamba 논문 리뷰", Mamba 블록 아키텍처) is: a projection to x and
z, a causal depthwise convolution with SiLU, a projection to B | C | dt, the
step size as the softplus of dt_proj (with its bias), the selective SSM, the
D skip, the SiLU(z) gate and the output projection.  Here:
  * the causal convolution of each channel is an explicit lower-triangular
    Toeplitz matrix T[t, s] = w[s - t + k - 1] (0 <= t - s < k), the newest
    input meeting the last tap;
  * the SSM is the quadratic form of the dual (convolution) mode (SSM의 이중
    연산 모드, with the zero-order hold of 이산화): y = M x per channel with
    M[t, s] = sum_n C_t[n] exp(A_n (S_t - S_s)) Bbar_s[n] for s <= t, where
    S_t is the running sum of the step sizes and
    Bbar_s[n] = expm1(delta_s A_n) / A_n * B_s[n];
  * softplus and SiLU are written out (log(1 + e^v), v / (1 + e^-v)).
No recurrence and no convolution routine appear, so the pin shares no
structure with the oracle's per-row loop.  Each of the block oracle's
test-only mistakes fails B1.
"""
import numpy as np
import pytest

import oracle
import synth


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _softplus(v):
    return np.logaddexp(0.0, v)


def _matrix_block(inp, io, N, R):
    f = lambda k: synth.to_f64(inp[k], io) if k in ("u", "W_in", "W_x", "W_dt", "W_out") \
        else np.asarray(inp[k], np.float64)
    u, W_in, W_x, W_dt, W_out = f("u"), f("W_in"), f("W_x"), f("W_dt"), f("W_out")
    cw, cb, bdt, A, Dk = f("conv_w"), f("conv_b"), f("b_dt"), f("A"), f("D")
    batch, L, M = u.shape
    E, K = cw.shape
    xz = np.einsum("blm,jm->blj", u, W_in)
    x, z = xz[..., :E], xz[..., E:]
    # causal depthwise convolution: one Toeplitz matrix per channel
    lag = np.arange(L)[:, None] - np.arange(L)[None, :]            # t - s
    tap = np.clip(K - 1 - lag, 0, K - 1)
    T = np.where((lag >= 0) & (lag < K), cw[:, tap], 0.0)           # (E, L, L)
    xc = _silu(np.einsum("ets,bse->bte", T, x) + cb)
    xd = np.einsum("ble,je->blj", xc, W_x[:2 * N + R])
    Bm, Cm, dt = xd[..., :N], xd[..., N:2 * N], xd[..., 2 * N:]
    delta = _softplus(np.einsum("blr,er->ble", dt, W_dt) + bdt)      # (batch, L, E)
    S = np.cumsum(delta, axis=1)                                     # running sum of delta
    y = np.empty_like(xc)
    causal = lag >= 0
    for b in range(batch):
        for e in range(E):
            decay = np.exp(A[e][None, None, :] * (S[b, :, e][:, None, None] - S[b, :, e][None, :, None]))
            bbar = np.expm1(delta[b, :, e][:, None] * A[e]) / A[e] * Bm[b]   # (L, N)
            Mts = np.einsum("tn,tsn,sn->ts", Cm[b], np.where(causal[..., None], decay, 0.0), bbar)
            y[b, :, e] = Mts @ xc[b, :, e]
    y = (y + Dk * xc) * _silu(z)
    return np.einsum("ble,me->blm", y, W_out)


CASES = [("f32", 2, 13, 8, 12, 4, 2, 4), ("bf16", 1, 20, 16, 24, 8, 1, 4), ("f32", 2, 9, 8, 16, 16, 3, 3)]


def _spec(io, batch, L, M, E, N, R, K):
    return synth.block_spec(synth.BLOCK2_8B, batch=batch, seqlen=L, d_model=M, d_inner=E, dstate=N, dt_rank=R,
                            d_conv=K, io=io)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_b%d_l%d_m%d_e%d_n%d_r%d_k%d" % c)
def test_b1_matrix_form_block(case):
    spec = _spec(*case)
    inp = synth.block_inputs(spec, 1)
    got = oracle.mamba_block(inp, spec.io, spec.dstate, spec.dt_rank)
    ref = _matrix_block(inp, spec.io, spec.dstate, spec.dt_rank)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("mutation", sorted(oracle.BLOCK_MUTATIONS))
def test_block_mutation_caught(mutation):
    spec = _spec(*CASES[0])
    inp = synth.block_inputs(spec, 1)
    got = oracle.mamba_block(inp, spec.io, spec.dstate, spec.dt_rank, mutation=mutation)
    ref = _matrix_block(inp, spec.io, spec.dstate, spec.dt_rank)
    assert not np.allclose(got, ref, rtol=1e-10, atol=1e-10), oracle.BLOCK_MUTATIONS[mutation]
