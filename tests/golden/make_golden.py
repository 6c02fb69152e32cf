"""Writes tiny_step_digests.txt from the CPU oracle only.

Run from the repository root:  python -m tests.golden.make_golden
"""
import os

import oracle
from tests.golden import HERE
from tests.test_oracle_e2e import tiny_step_digests


def main():
    oracle.lib()
    dig = tiny_step_digests(oracle)
    path = os.path.join(HERE, "tiny_step_digests.txt")
    with open(path, "w") as f:
        f.write("# SHA-256 prefixes of the oracle's outputs for the tiny training step\n")
        f.write("# (X 64x256, W 128x256, no rotation, SGD lr 1e-3, seed 0, step 0).\n")
        f.write("# Written by tests/golden/make_golden.py, which calls only oracle/.\n")
        for k, v in dig.items():
            f.write(f"{k} {v}\n")
    print(open(path).read())


if __name__ == "__main__":
    main()
