"""One Mamba block forward on MI355X: the projections are hipBLASLt GEMMs
(through torch.mm on contiguous bf16 operands); the causal conv + SiLU and the
selective scan (with the softplus step size, D skip and SiLU(z) gate fused)
are this library's kernels (``causal_conv1d``, ``selective_scan_fwd``).

Order of the block ("Mamba 논문 리뷰", tildalice.io, Mamba 블록 아키텍처 and the
SelectiveSSM listing): in_proj to x and z; Conv1D + SiLU on x; x_proj to
B | C | dt; dt_proj (with bias, softplus applied in the scan); the selective
scan; y * SiLU(z); out_proj.
"""
from __future__ import annotations

import torch

from . import causal_conv1d, selective_scan_fwd


class BlockWeights:
    """Device weights of one block.  Projection weights are stored transposed
    ((in, out), contiguous) so each projection is one plain GEMM."""

    def __init__(self, host: dict, dstate: int, dt_rank: int, device="cuda"):
        bf = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16) if a.dtype.name == "uint16" \
            else torch.from_numpy(a)
        t = lambda k: bf(host[k]).to(device).t().contiguous()
        f = lambda k: torch.from_numpy(host[k]).to(device).contiguous()
        self.W_in_t, self.W_x_t, self.W_dt_t, self.W_out_t = t("W_in"), t("W_x"), t("W_dt"), t("W_out")
        self.conv_w, self.conv_b, self.b_dt, self.A, self.D = f("conv_w"), f("conv_b"), f("b_dt"), f("A"), f("D")
        self.N, self.R = dstate, dt_rank
        self.E = self.W_in_t.shape[1] // 2
        self.M = self.W_in_t.shape[0]


def mamba_block_fwd(u: torch.Tensor, w: BlockWeights, mark=None) -> torch.Tensor:
    """u: (batch, L, d_model) bf16 -> (batch, L, d_model) bf16.  `mark`, if
    given, is called after each stage (for timing)."""
    batch, L, M = u.shape
    E, N, R = w.E, w.N, w.R
    T = batch * L
    xz = torch.mm(u.reshape(T, M), w.W_in_t).view(batch, L, 2 * E)       # in_proj
    if mark: mark("in_proj")
    x, z = xz[..., :E], xz[..., E:]
    xc = causal_conv1d(x, w.conv_w, w.conv_b, silu=True)                 # conv + SiLU
    if mark: mark("conv")
    xd = torch.mm(xc.view(T, E), w.W_x_t)                               # x_proj: B | C | dt | padding
    delta = torch.mm(xd[:, 2 * N:2 * N + R], w.W_dt_t).view(batch, L, E)  # dt_proj (bias in the scan)
    if mark: mark("x_proj+dt_proj")
    xd = xd.view(batch, L, -1)
    y, _ = selective_scan_fwd(xc, delta, w.A, xd[..., :N], xd[..., N:2 * N], D=w.D, z=z,
                              delta_softplus=True, delta_bias=w.b_dt)
    if mark: mark("scan")
    out = torch.mm(y.view(T, E), w.W_out_t).view(batch, L, M)           # out_proj
    if mark: mark("out_proj")
    return out
