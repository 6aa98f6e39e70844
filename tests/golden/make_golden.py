"""Writes the stored tile list of the tiny workload (512 tokens, documents
[64, 192, 32, 224], one call with Q = KV = the whole sequence, 128x64 tiles).

It calls only the oracle planner and the seeded workload description.
Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as W  # noqa: E402
from oracle import planner as P  # noqa: E402


def main():
    w = W.tiny()
    pl = P.plan(w.cu, w.q_segs, w.steps[0].kv_segs, 128, 64)
    with open(os.path.join(HERE, "tiny_tiles_128x64.txt"), "w") as f:
        f.write("# q_tile kv_tile class(0=FULL,1=DIAGONAL,2=PARTIAL); documents [64,192,32,224], BM=128 BN=64\n")
        f.write("# written by tests/golden/make_golden.py from the oracle planner\n")
        for a, b, c in zip(pl.q_tile, pl.kv_tile, pl.cls):
            f.write(f"{a} {b} {c}\n")


if __name__ == "__main__":
    main()
