"""Write workload0_oracle.txt: the oracle's outputs on the tiny fp32 workload.

Calls only the oracle and the seeded input generator.  Run from the repo root:
    python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload0_oracle.txt")


def input_digest(x):
    h = hashlib.sha256()
    for k in ("u", "delta", "A", "B", "C", "D", "z", "dt_bias"):
        h.update(x[k].contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def main():
    x = gen.scan_inputs(0)
    y, last = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["dt_bias"], True)
    with open(OUT, "w") as f:
        f.write("# tiny fp32 workload: B=1 D=16 N=4 L=64, seed 0; oracle y [1,16,64] then last_state [1,16,4]\n")
        f.write(f"input_sha256 {input_digest(x)}\n")
        for v in y.ravel():
            f.write(f"y {float(v)!r}\n")
        for v in last.ravel():
            f.write(f"last {float(v)!r}\n")


if __name__ == "__main__":
    main()
