"""Build the CPU oracle library (test infrastructure only).

Compiles ``tgemm_ref.c`` with gcc into ``liboracle_tgemm.so`` next to this
file. Plain ``-O2`` with OpenMP; no fast-math and no floating-point
contraction, so every element is the literal ascending-k fp64 sum.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tgemm_ref.c")
LIB = os.path.join(HERE, "liboracle_tgemm.so")


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB) -> str:
    """sanitize: AddressSanitizer and UndefinedBehaviorSanitizer instrumentation
    (for the sanitizer test tier; load the result with libasan preloaded)."""
    tmp = out + ".tmp"
    san = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"] if sanitize else []
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", *san,
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
