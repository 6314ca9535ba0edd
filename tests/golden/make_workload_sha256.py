"""Write workload_sha256.txt: the SHA-256 of each benchmark workload's seeded
operands (A, then B in its stored layout) as binary16 bytes, with the numpy
version that produced them. Calls only the input generator.

    python tests/golden/make_workload_sha256.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from dense_tiled_gemm_tgemm_amd import inputs  # noqa: E402


def main():
    lines = [f"# numpy {np.__version__}; name sha256(A) sha256(B)"]
    for name, w in inputs.WORKLOADS.items():
        A, B = inputs.make_inputs(w)
        lines.append(f"{name} {inputs.sha256(A)} {inputs.sha256(B)}")
    with open(os.path.join(HERE, "workload_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
