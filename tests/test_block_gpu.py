"""GPU parity of one Mamba block forward (hipBLASLt projections + this
library's conv and scan kernels) against the fp64 oracle composition.

Every intermediate on the GPU is bf16 (the GEMM outputs, the conv output, the
scan output), so the block output meets the bf16 bound, rel-L2 <= 2e-2.
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

from selective_state_space_60_amd.block import BlockWeights, mamba_block_fwd  # noqa: E402


def _check(spec, seed):
    banner("block %s seed %d" % (spec.name, seed))
    inp = synth.block_inputs(spec, seed)
    w = BlockWeights(inp, spec.dstate, spec.dt_rank)
    out = mamba_block_fwd(dev_tensor(inp["u"], "bf16"), w)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16 and out.shape == (spec.batch, spec.seqlen, spec.d_model)
    ref = oracle.mamba_block(inp, "bf16", spec.dstate, spec.dt_rank)
    assert_close(host_f64(out), ref, "bf16", spec.name + " out")


@pytest.mark.parametrize("case", [(2, 300, 64, 128, 16, 1, 4), (1, 129, 96, 192, 16, 4, 4), (3, 70, 32, 64, 8, 2, 3)],
                         ids=lambda c: "b%d_l%d_m%d_e%d_n%d_r%d_k%d" % c)
def test_block_small(case):
    batch, L, M, E, N, R, K = case
    spec = synth.block_spec(synth.BLOCK2_8B, batch=batch, seqlen=L, d_model=M, d_inner=E, dstate=N, dt_rank=R,
                            d_conv=K)
    _check(spec, 1)


def test_block_2_8b_width():
    """The 2.8B block's full width (d_model 2560, E 5120, N 16, rank 1) on a
    shorter batch (1 x 1024 tokens), every output."""
    _check(synth.block_spec(synth.BLOCK2_8B, batch=1, seqlen=1024), 2)
