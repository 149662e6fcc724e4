"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, binary32 semantics pinned: -ffp-contract=off keeps every a*b+c as
two rounded operations, and no -ffast-math (which would also flush subnormals).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, f) for f in ("nvfp4_oracle.c", "mxfp4_oracle.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-o", LIB + ".tmp", *SRCS, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
