"""How much the bf16 storage of the SSD's inter-chunk state adds to y's error.

The chunk scan takes the state entering each chunk (S_in) as a bf16 matrix-core
operand, while the state passing keeps it in fp32.  The inter-chunk output
term (obsidian-dorae222 "Mamba-2", SSD 타일링 알고리즘: exp(A_cum_i) C_i . S_in[c])
is linear in S_in, so the error that rounding S_in to bf16 adds to y is
exactly exp(A_cum_i) C_i (S_in_bf16 - S_in)^T.  This test measures it with the
fp64 chunked oracle on the 2.7B-shaped layer's distributions (fewer heads, the
same per-head statistics) and holds it well below the rounding of y itself to
bf16, which every bf16-output path pays anyway.
"""
import numpy as np
import pytest

import oracle
import synth


def _bf16_round(a):
    """float64 -> float32 -> bf16 (round to nearest even) -> float64."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("heads,seqlen", [(8, 4096), (16, 2048)])
def test_bf16_state_operand_error_share(heads, seqlen):
    q = synth.ssd_spec(synth.SSD2_7B, batch=1, seqlen=seqlen, nheads=heads)
    inp = synth.ssd_inputs(q, 0)
    r = oracle.ssd_chunked(inp, "bf16", q.chunk)
    y, A_cum, S_in = r["y"], r["A_cum"], r["S_in"]       # A_cum (b, H, L); S_in (b, nc, H, P, N)
    C = synth.to_f64(inp["C"], "bf16")[:, :, 0]           # one group: (b, L, N)
    dS = _bf16_round(S_in) - S_in
    dy = np.zeros_like(y)
    for c in range(S_in.shape[1]):
        s, e = c * q.chunk, min(seqlen, (c + 1) * q.chunk)
        decay = np.exp(np.transpose(A_cum[:, :, s:e], (0, 2, 1)))     # (b, q, H)
        dy[:, s:e] = decay[..., None] * np.einsum("bhpn,bin->bihp", dS[:, c], C[:, s:e])
    ny = np.linalg.norm(y)
    share = np.linalg.norm(dy) / ny
    y_round = np.linalg.norm(_bf16_round(y) - y) / ny
    print("S_in bf16: rel-L2 %.3e of y; y rounded to bf16: %.3e" % (share, y_round))
    assert 0 < share <= 0.2 * y_round
