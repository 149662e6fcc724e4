"""Build the two sanitizer programs: the CPU reference (oracle/*.c) driven by
oracle_driver.c, and libnvfp4's C-ABI validation layer (nvfp4_api.cpp) on
host stubs driven by api_driver.cpp, each with AddressSanitizer and
UndefinedBehaviorSanitizer (no recovery: the first report aborts).  Host
compilers only (gcc / g++); no GPU code is built here."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "bit_microscaled_numerics_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ORACLE = os.path.join(HERE, "oracle_asan")
API = os.path.join(HERE, "api_asan")
ORACLE_LIB = os.path.join(HERE, "liboracle_asan.so")


def build() -> tuple[str, str]:
    cc = ["gcc", *SAN, "-fopenmp", "-ffp-contract=off", "-std=gnu11", "-Wall",
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "nvfp4_oracle.c"),
          os.path.join(ROOT, "oracle", "mxfp4_oracle.c"), "-lm", "-o", ORACLE]
    subprocess.run(cc, check=True)
    cxx = ["g++", *SAN, "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(HERE, "api_driver.cpp"), os.path.join(HERE, "api_stubs.cpp"),
           os.path.join(CSRC, "nvfp4_api.cpp"), "-o", API]
    subprocess.run(cxx, check=True)
    so = ["gcc", *SAN, "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
          os.path.join(ROOT, "oracle", "nvfp4_oracle.c"),
          os.path.join(ROOT, "oracle", "mxfp4_oracle.c"), "-lm", "-o", ORACLE_LIB]
    subprocess.run(so, check=True)
    return ORACLE, API


def preload() -> str:
    """The sanitizer runtimes a Python process needs preloaded to load
    ORACLE_LIB."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                             check=True).stdout.strip()
        libs.append(os.path.realpath(out))
    return ":".join(libs)


if __name__ == "__main__":
    print(build())
