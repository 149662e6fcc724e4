"""Loader of the test-only helper library (tests/devhelpers/devtest.hip):
the NVFP4 kernels' device helpers on arrays, plus the value sets the tests
run them over.  Building the library compiles the helpers from the kernels'
own headers; nothing here computes a code."""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "devhelpers", "libnvfp4_devtest.so")
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        from devhelpers import build
        build.build()
    lib = ctypes.CDLL(LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    for name, args in {"devtest_e4m3_code": [vp, vp, i64, vp],
                       "devtest_encode_rtn": [vp, vp, i64, vp],
                       "devtest_encode_sr": [vp, vp, vp, i64, vp],
                       "devtest_block_scale": [vp, i64, ctypes.c_float, vp, vp, vp],
                       "devtest_gemm_decode": [vp, vp, vp, vp, vp, i64, vp]}.items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, ctypes.c_int
    lib.devtest_sr_value_host.argtypes = [vp, vp, vp, i64]
    lib.devtest_sr_value_host.restype = None
    _lib = lib
    return lib


def sr_value_host(v: np.ndarray, u: np.ndarray) -> np.ndarray:
    """The kernels' stochastic-rounding decision compiled for the CPU: the E2M1
    grid value (sign of v kept) chosen for v with random bits u."""
    v = np.ascontiguousarray(v, np.float32)
    u = np.ascontiguousarray(np.broadcast_to(u, v.shape), np.uint16)
    out = np.empty(v.shape, np.float32)
    load().devtest_sr_value_host(v.ctypes.data, u.ctypes.data, out.ctypes.data, v.size)
    return out


def f32(bits) -> np.ndarray:
    return np.asarray(bits, np.uint32).view(np.float32)


# Points where the E2M1 decision changes: the grid values (SR's carry
# boundaries) and the midpoints between them (RTN's), plus the ends.
E2M1_GRID = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E2M1_MID = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def near(points, ulps: int = 16) -> np.ndarray:
    """Every binary32 within `ulps` patterns of each point (non-negative)."""
    out = []
    for p in points:
        b = int(np.float32(p).view(np.uint32))
        out.append(np.arange(max(b - ulps, 0), b + ulps + 1, dtype=np.uint32))
    return f32(np.unique(np.concatenate(out)))


def sr_near_points() -> np.ndarray:
    """The SR test values near every decision point (and 0, 8, one binade
    below 0.25), both signs."""
    v = near(E2M1_GRID + E2M1_MID + [0.0, 0.125, 8.0])
    return np.concatenate([v, -v])


def sr_strided_values(stride: int = 4099) -> np.ndarray:
    """Every `stride`-th binary32 pattern in [0, 8], alternating signs."""
    v = f32(np.arange(0, 0x41000000 + 1, stride, dtype=np.uint32))
    s = np.where(np.arange(v.size) % 2 == 1, np.float32(-1), np.float32(1))
    return (v * s).astype(np.float32)
