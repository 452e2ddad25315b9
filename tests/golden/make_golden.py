"""Write the oracle's outputs for the tiny fp32 workload (batch 1, L 64, dim 16,
N 4, seed 0) as a text fixture. Calls only ``oracle`` and ``ssm_inputs``.

The pages print no numeric worked example of the scan, so this fixture is not a
pin of the oracle: it freezes the oracle's answer so that any later change to
its arithmetic shows up as a diff of this file in the same commit.

Usage: python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import ssm_inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.txt")


def main():
    x = ssm_inputs.scan_inputs(ssm_inputs.CONFIGS["tiny"], seed=0)
    y, hl = oracle.load().selective_scan(**x)
    with open(OUT, "w") as f:
        f.write("# oracle y (1,64,16) then h_last (1,16,4), tiny fp32 workload, seed 0\n")
        f.write("# written by tests/golden/make_golden.py\n")
        for v in np.concatenate([y.ravel(), hl.ravel()]):
            f.write("%.17g\n" % v)


if __name__ == "__main__":
    main()
