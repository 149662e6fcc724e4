"""Build the test-only helper library libnvfp4_devtest.so (devtest.hip):
the NVFP4 kernels' device helpers on arrays, for the tests that compare them
with the CPU reference.  Same compiler flags as libnvfp4.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libnvfp4_devtest.so")

if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def build(verbose: bool = False) -> str:
    from bit_microscaled_numerics_amd import build as libbuild
    cmd = ["hipcc", "-x", "hip", *libbuild.CFLAGS, f"-I{libbuild.CSRC}", "-shared",
           os.path.join(HERE, "devtest.hip"), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
