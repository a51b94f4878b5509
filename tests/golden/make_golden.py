"""Write the oracle regression fixtures in this folder.

The pages print no worked numeric example for FAVOR+, so no stored value here
comes from the pages.  These fixtures are regression values of the oracle
itself (fp64, CPU), written by this script, which calls only ``oracle`` and
the seeded input generator ``workloads``.  They guard the oracle against
silent drift; the oracle's correctness is pinned separately by
tests/test_oracle_pins.py.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402

ROWS = [0, 1, 17, 128, 255]


def main():
    w = workloads.workload("tiny_f32")
    W = oracle.draw_w(w.seed_w, w.m, w.d).astype(np.float32)
    Q, K, V = (t.double().numpy()[0, 0] for t in workloads.host_qkv(w))
    Wd = W.astype(np.float64)
    ob = oracle.bidir(Q, K, V, Wd)
    oc = oracle.causal(Q, K, V, Wd)
    with open(os.path.join(HERE, "tiny_f32_W.txt"), "w") as f:
        f.write(f"# oracle.draw_w(seed={w.seed_w}, m={w.m}, d={w.d}) rounded to fp32, row-major\n")
        for r in W:
            f.write(" ".join(f"{x:.9e}" for x in r) + "\n")
    for name, o in (("bidir", ob), ("causal", oc)):
        with open(os.path.join(HERE, f"tiny_f32_{name}_rows.txt"), "w") as f:
            f.write(f"# oracle.{name} on the tiny_f32 workload (seed_in={w.seed_in}) with the W above;"
                    f" rows {ROWS}, fp64\n")
            for i in ROWS:
                f.write(f"{i} " + " ".join(f"{x:.17e}" for x in o[i]) + "\n")


if __name__ == "__main__":
    main()
