"""Write the oracle's float64 outputs for the tiny fp32 workload (seed 0).

Calls only the oracle and the seeded input generator.  The fixture guards the
oracle against silent change: a later edit to its arithmetic must reproduce
these values or regenerate them in a commit that names the reason.
The pages print no numeric worked example for this pass, so no fixture here
carries a value from them.

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from linear_recurrent_sequence_amd import workloads  # noqa: E402


def main():
    x = workloads.make("tiny_fp32", seed=0)
    h, m, n = oracle.forward_stabilized(x["q"], x["k"], x["v"], x["igate"], x["fgate"])
    path = os.path.join(HERE, "tiny_fp32_seed0.txt")
    with open(path, "w") as f:
        f.write("# oracle.forward_stabilized on workloads.make('tiny_fp32', seed=0)\n")
        f.write("# B=1 NH=1 T=64 d=16; one line per t: m n h[0..15] (float64, repr)\n")
        for t in range(64):
            vals = [m[0, 0, t], n[0, 0, t]] + list(h[0, 0, t])
            f.write(" ".join(repr(float(v)) for v in vals) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
