"""Build the CPU oracle shared library (test infrastructure only).

gcc, -O2, no fast-math, -ffp-contract=off so that no multiply-add is fused:
every float operation in the oracle is one IEEE single (or double) rounding.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q8kv_oracle.c")
LIB = os.path.join(HERE, "liboracle_q8kv.so")

FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
         "-Wall", "-Wextra", "-fPIC", "-shared"]


def build(verbose=False):
    """Compile the oracle into oracle/liboracle_q8kv.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc"] + FLAGS + [SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
