"""Pin of the oracle's Mamba block composition (oracle.mamba_block).

B1: an independent float64 torch implementation of the block, written here
from the definitions.  These are the block figure and listing of
tildalice.io "Mamba 논문 리뷰" (in_proj to 2E, depthwise causal Conv1D with
k - 1 steps of padding cut back to L, SiLU, x_proj to B | C | dt, dt_proj with
bias and softplus, the selective scan with zero-order hold from the 이산화
section, D skip, SiLU(z) gate, out_proj).  Its scan is a dense per-step loop
over the full (E, N) state in torch, unrelated to the C oracle's per-row
loop.  Each of the block oracle's test-only mistakes fails B1.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def _torch_block(inp, io, N, R):
    t = lambda k: torch.from_numpy(synth.to_f64(inp[k], io)) if k in ("u", "W_in", "W_x", "W_dt", "W_out") \
        else torch.from_numpy(np.asarray(inp[k], np.float64))
    u, W_in, W_x, W_dt, W_out = t("u"), t("W_in"), t("W_x"), t("W_dt"), t("W_out")
    cw, cb, bdt, A, Dk = t("conv_w"), t("conv_b"), t("b_dt"), t("A"), t("D")
    batch, L, M = u.shape
    E, K = cw.shape
    xz = F.linear(u, W_in)
    x, z = xz[..., :E], xz[..., E:]
    conv = torch.nn.Conv1d(E, E, K, padding=K - 1, groups=E, dtype=torch.float64)
    with torch.no_grad():
        conv.weight.copy_(cw[:, None, :])
        conv.bias.copy_(cb)
        xc = F.silu(conv(x.transpose(1, 2))[..., :L].transpose(1, 2))
    xd = F.linear(xc, W_x[:2 * N + R])
    Bm, Cm, dt = xd[..., :N], xd[..., N:2 * N], xd[..., 2 * N:]
    delta = F.softplus(F.linear(dt, W_dt, bdt))               # (batch, L, E)
    dA = torch.exp(delta[..., None] * A)                       # (batch, L, E, N)
    dB = torch.expm1(delta[..., None] * A) / A * Bm[:, :, None, :]
    h = torch.zeros(batch, E, N, dtype=torch.float64)
    ys = []
    for s in range(L):
        h = dA[:, s] * h + dB[:, s] * xc[:, s, :, None]
        ys.append((h * Cm[:, s, None, :]).sum(-1))
    y = (torch.stack(ys, 1) + Dk * xc) * F.silu(z)
    return F.linear(y, W_out).detach().numpy()


CASES = [("f32", 2, 13, 8, 12, 4, 2, 4), ("bf16", 1, 20, 16, 24, 8, 1, 4), ("f32", 2, 9, 8, 16, 16, 3, 3)]


def _spec(io, batch, L, M, E, N, R, K):
    return synth.block_spec(synth.BLOCK2_8B, batch=batch, seqlen=L, d_model=M, d_inner=E, dstate=N, dt_rank=R,
                            d_conv=K, io=io)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s_b%d_l%d_m%d_e%d_n%d_r%d_k%d" % c)
def test_b1_independent_torch_block(case):
    spec = _spec(*case)
    inp = synth.block_inputs(spec, 1)
    got = oracle.mamba_block(inp, spec.io, spec.dstate, spec.dt_rank)
    ref = _torch_block(inp, spec.io, spec.dstate, spec.dt_rank)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("mutation", sorted(oracle.BLOCK_MUTATIONS))
def test_block_mutation_caught(mutation):
    spec = _spec(*CASES[0])
    inp = synth.block_inputs(spec, 1)
    got = oracle.mamba_block(inp, spec.io, spec.dstate, spec.dt_rank, mutation=mutation)
    ref = _torch_block(inp, spec.io, spec.dstate, spec.dt_rank)
    assert not np.allclose(got, ref, rtol=1e-10, atol=1e-10), oracle.BLOCK_MUTATIONS[mutation]
