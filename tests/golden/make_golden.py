"""Writes tests/golden/tiny_scan_oracle.txt: the oracle's output for the tiny
fp32 workload (batch 1, L 64, D 4, N 4, seed 0).  Calls only oracle/ and
synth/.  The file is a regression fixture for the oracle itself; its values
are pinned to the pages through the tests in test_oracle_pins.py."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    inp = synth.scan_inputs(synth.TINY, 0)
    y, h = oracle.selective_scan(inp, "f32")
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_scan_oracle.txt")
    with open(out, "w") as f:
        f.write("# oracle y[0, t, d] and h_last[0, d, n] for %s, seed 0 (fp64, %%.17g)\n" % synth.TINY.name)
        for t in range(y.shape[1]):
            f.write("y %d " % t + " ".join("%.17g" % v for v in y[0, t]) + "\n")
        for d in range(h.shape[1]):
            f.write("h %d " % d + " ".join("%.17g" % v for v in h[0, d]) + "\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
