"""The stochastic-rounding decision of the HIP encoders, compiled for the CPU
from the kernels' own source (e2m1_sr_twice in nvfp4_device.h, which returns
twice the chosen value for the FP4 encode's scale of 2; halved here), against the
CPU reference's definition: between the neighbouring E2M1 values lo <= |v| <
hi, round away from zero iff the 16 random bits u < (|v| - lo)/(hi - lo) *
65536 ("NVFP4 Trains with Precision of 16-Bit and Speed and Efficiency of
4-Bit", stochastic-rounding section: the larger neighbour with probability
given by the distance).  The kernels take the decision as an add-and-carry on
the binary32 bits from 1 up and as a ceiling of a fused multiply-add below
1, where the grid step is uniform; the values here
are every binary32 within 16 patterns of every grid value and midpoint (and
of 0, 0.125, 8) with all 65536 random values, and every 4099th binary32 in
[0, 8] with every 97th random value.  CPU only."""
import numpy as np

import oracle
import devtest

E2M1 = np.array([oracle.e2m1_decode(c) for c in range(16)], np.float32)


def _check(v: np.ndarray, u: np.ndarray):
    got = devtest.sr_value_host(v, u)
    want = E2M1[oracle.e2m1_sr(v, u)]
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, (f"{bad.size} mismatches, first v={v[bad[0]]!r} "
                           f"({v[bad[0]:bad[0] + 1].view(np.uint32)[0]:#010x}) u={u[bad[0]]} "
                           f"kernel={got[bad[0]]} reference={want[bad[0]]}")


def test_near_every_decision_point_all_random_values():
    v = devtest.sr_near_points()
    u = np.arange(65536, dtype=np.uint16)
    for i in range(0, v.size, 64):
        vv = v[i:i + 64]
        _check(np.repeat(vv, u.size), np.tile(u, vv.size))


def test_strided_values_strided_random_values():
    v = devtest.sr_strided_values(4099)
    u = np.arange(0, 65536, 97, dtype=np.uint16)
    for i in range(0, v.size, 16384):
        vv = v[i:i + 16384]
        _check(np.repeat(vv, u.size), np.tile(u, vv.size))


def test_saturation_and_non_grid_magnitudes():
    """|v| above 6 gives +-6; the chosen value is always a neighbour of |v|."""
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(6, 1e4, 4096), -rng.uniform(6, 1e4, 4096)]).astype(np.float32)
    u = rng.integers(0, 65536, v.size).astype(np.uint16)
    got = devtest.sr_value_host(v, u)
    assert np.array_equal(np.abs(got), np.full(v.size, 6.0, np.float32))
    assert np.array_equal(np.signbit(got), np.signbit(v))
    _check(v, u)
