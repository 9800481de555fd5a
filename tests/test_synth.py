"""The seeded input generator: determinism, slice addressability, the mixer
against its published definition, and bf16 rounding against hand-computed
bit patterns."""
import struct

import numpy as np
import pytest

import synth

MASK = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def _mix(z):
    # SplitMix64 finaliser (Steele, Lea, Flood, OOPSLA 2014), in Python integers
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def test_splitmix64_matches_definition():
    seed, stream = 5, 3
    key = _mix(_mix((seed * GAMMA + 0x2545F4914F6CDD1D) & MASK) ^ ((stream * 0xD1B54A32D192ED03) & MASK))
    got = synth.raw(6, 10, seed, stream)
    want = [_mix((key + (i + 1) * GAMMA) & MASK) for i in range(10, 16)]
    assert [int(v) for v in got] == want


def test_deterministic_and_sliceable():
    d = synth.Dist(synth.NORMAL, 0.0, 1.0)
    a = synth.fill((1000,), d, "f32", 7, 1)
    b = synth.fill((1000,), d, "f32", 7, 1)
    assert np.array_equal(a, b)
    part = synth.fill((300,), d, "f32", 7, 1, start=500)
    assert np.array_equal(part, a[500:800])
    assert not np.array_equal(synth.fill((1000,), d, "f32", 7, 2), a)
    assert not np.array_equal(synth.fill((1000,), d, "f32", 8, 1), a)
    # threaded fill of a large tensor equals the single-call slice
    big = synth.fill((3_000_000,), d, "bf16", 1, 4)
    assert np.array_equal(big[2_000_000:2_000_100], synth.fill((100,), d, "bf16", 1, 4, start=2_000_000))


def _bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def _f(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


@pytest.mark.parametrize("fbits,want", [
    (0x3F800000, 0x3F80),  # 1.0
    (0x3F808000, 0x3F80),  # 1 + 2^-8: exact tie, upper half even -> down
    (0x3F818000, 0x3F82),  # tie with odd upper half -> up
    (0x3F808001, 0x3F81),  # just above the tie -> up
    (0x3F807FFF, 0x3F80),  # just below the tie -> down
    (0xC0200000, 0xC020),  # -2.5
    (0x7F800000, 0x7F80),  # +inf
    (0x7F7FFFFF, 0x7F80),  # FLT_MAX rounds to +inf
    (0x00000001, 0x0000),  # smallest denormal -> +0
])
def test_bf16_round_to_nearest_even(fbits, want):
    assert synth.f32_to_bf16_bits(_f(fbits)) == want


def test_bf16_nan_stays_nan():
    b = synth.f32_to_bf16_bits(float("nan"))
    assert (b & 0x7F80) == 0x7F80 and (b & 0x007F) != 0


def test_distributions():
    n = 1 << 20
    z = synth.fill((n,), synth.Dist(synth.NORMAL, 0.0, 1.0), "f32", 0, 1).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    sp = synth.fill((n,), synth.Dist(synth.SOFTPLUS_NORMAL, -3.0, 1.0), "f32", 0, 2).astype(np.float64)
    v = synth.fill((n,), synth.Dist(synth.NORMAL, -3.0, 1.0), "f32", 0, 2).astype(np.float64)
    assert np.all(sp > 0)
    assert np.allclose(sp, np.log1p(np.exp(v)), rtol=1e-6)
    A = synth.fill((8, 16), synth.Dist(synth.NEG_IDX, period=16), "f32", 0, 3)
    assert np.array_equal(A, -np.tile(np.arange(1, 17, dtype=np.float32), (8, 1)))
    ne = synth.fill((n,), synth.Dist(synth.NEG_EXP_UNIFORM, 0.0, 2.7), "f32", 0, 3)
    assert ne.max() <= -1.0 and ne.min() >= -np.exp(2.7) * (1 + 1e-6)


def test_workload_shapes():
    inp = synth.scan_inputs(synth.TINY, 0)
    assert inp["x"].shape == (1, 64, 4) and inp["B"].shape == (1, 64, 4) and inp["A"].shape == (4, 4)
    assert "z" not in inp and inp["D"].shape == (4,)
    s = synth.ssd_spec(synth.SSD2_7B, batch=1, seqlen=8, nheads=4)
    d = synth.ssd_inputs(s, 0)
    assert d["x"].shape == (1, 8, 4, 64) and d["B"].shape == (1, 8, 1, 64) and d["delta"].shape == (1, 8, 4)
    assert synth.MAMBA2_8B.algorithmic_bytes() == 4 * 4096 * 5120 * 8 + 4 * 4096 * 64 + 5120 * 16 * 4 + 5120 * 4


def test_oracle_regression_golden():
    """The oracle still reproduces its stored tiny-workload output (written by
    tests/golden/make_golden.py)."""
    import os
    import oracle
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_scan_oracle.txt")
    ys, hs = {}, {}
    for line in open(path):
        if line.startswith("#"):
            continue
        tag, i, *vals = line.split()
        (ys if tag == "y" else hs)[int(i)] = [float(v) for v in vals]
    y, h = oracle.selective_scan(synth.scan_inputs(synth.TINY, 0), "f32")
    assert np.array_equal(y[0], np.array([ys[t] for t in range(len(ys))]))
    assert np.array_equal(h[0], np.array([hs[d] for d in range(len(hs))]))
