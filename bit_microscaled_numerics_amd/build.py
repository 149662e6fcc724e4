"""Build libnvfp4.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Flags that fix the numerics: -ffp-contract=off (no fused multiply-add, so
the quantizer's binary32 arithmetic is the reference's), no fast-math
(correctly rounded division, subnormals kept), and packed-FP32 instruction
selection disabled.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build", "nvfp4")
LIB = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["nvfp4_api.cpp", "nvfp4_quant.hip", "nvfp4_gemm.hip", "mxfp4.hip", "mfma_probe.hip"]
ARCH = os.environ.get("NVFP4_OFFLOAD_ARCH", "gfx950")

CFLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = ["hipcc", *lang, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
