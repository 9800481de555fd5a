"""ssm_selective_scan_fwd_noalloc: the selective scan with its workspace in the
library's static device scratch instead of a caller-owned buffer.

The GPU test calls it through the C ABI on problems whose sequence is cut into
segments (so the scratch is used), twice in a row with the second problem
smaller, and checks each output against ssm_selective_scan_fwd with a
caller-owned workspace (the same kernels: bit-identical) and against the fp64
oracle at the fp32 bar.  The CPU test checks that a problem whose workspace
exceeds the scratch is rejected before any HIP call.
"""
import ctypes

import numpy as np
import pytest

import selective_state_space_60_amd as ssm


def _desc_only(batch, L, D, N):
    """A valid fp32 descriptor and fake (never dereferenced) pointers."""
    def td(shape):
        d = ssm.TensorDesc()
        d.dtype, d.ndim = ssm.SSM_F32, len(shape)
        acc = 1
        for i in reversed(range(len(shape))):
            d.shape[i], d.stride[i] = shape[i], acc
            acc *= shape[i]
        return d
    d = ssm.ScanDesc()
    d.batch, d.seqlen, d.dim, d.dstate, d.flags = batch, L, D, N, 0
    shapes = {"x": (batch, L, D), "delta": (batch, L, D), "A": (D, N), "B": (batch, L, N), "C": (batch, L, N),
              "y": (batch, L, D)}
    p = ssm.ScanPtrs()
    for i, (k, sh) in enumerate(shapes.items()):
        setattr(d, k, td(sh))
        setattr(p, k, (i + 1) << 40)
    return d, p


def test_noalloc_rejects_workspace_beyond_scratch():
    """The 1M-token shape with 64 states plans more than 4 MiB of workspace:
    rejected with SSM_ERR_WORKSPACE before any HIP call (this runs without a
    GPU).  With 16 states the same shape fits."""
    d, p = _desc_only(1, 1 << 20, 1536, 64)
    assert ssm.selective_scan_workspace_size(d) > ssm.SCAN_STATIC_SCRATCH_BYTES
    assert ssm.lib().ssm_selective_scan_fwd_noalloc(ctypes.byref(d), ctypes.byref(p), None) == \
        ssm.SSM_ERR_WORKSPACE
    d, p = _desc_only(1, 1 << 20, 1536, 16)
    assert 0 < ssm.selective_scan_workspace_size(d) <= ssm.SCAN_STATIC_SCRATCH_BYTES


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_twice():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import oracle
    import synth
    from _gpu import assert_close, banner, dev_tensor, host_f64

    cases = [synth.scan_spec(synth.LONG1M, batch=1, seqlen=40000, dim=40, has_z=True, has_D=True),
             synth.scan_spec(synth.LONG1M, batch=1, seqlen=9000, dim=24, has_z=True, has_D=True)]
    for k, spec in enumerate(cases):
        banner("noalloc scan %s (call %d)" % (spec.name, k + 1))
        inp = synth.scan_inputs(spec, 7 + k)
        g = {n: dev_tensor(inp[n], spec.io) for n in ("x", "delta", "B", "C", "z")}
        g["A"], g["D"] = dev_tensor(inp["A"], "f32"), dev_tensor(inp["D"], "f32")
        desc = ssm.scan_desc(g["x"], g["delta"], g["A"], g["B"], g["C"], D=g["D"], z=g["z"], y=g["x"],
                             h_last=torch.empty(1, spec.dim, spec.dstate, device="cuda"))
        assert ssm.selective_scan_workspace_size(desc) > 0  # the sequence is split: the scratch is used
        args = (g["x"], g["delta"], g["A"], g["B"], g["C"])
        y0 = torch.empty_like(g["x"])
        y1 = torch.empty_like(g["x"])
        _, h0 = ssm.selective_scan_fwd(*args, D=g["D"], z=g["z"], y=y0, want_hlast=True)
        _, h1 = ssm.selective_scan_fwd_noalloc(*args, D=g["D"], z=g["z"], y=y1, want_hlast=True)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(h0, h1), "noalloc differs from the workspace entry point"
        yr, hr = oracle.selective_scan(inp, spec.io)
        assert_close(host_f64(y1), yr, spec.io, "noalloc y")
        assert_close(host_f64(h1), hr, spec.io, "noalloc h_last")
