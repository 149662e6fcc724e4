"""The matrix-core measurement probe on the GPU: sane throughput and clock
for every operand kind, and never above the published dense FP16 peak."""
import pytest

import bit_microscaled_numerics_amd as nv
from parity import say

pytestmark = pytest.mark.gpu

PEAK_FP16_TFLOPS = 2500.0


def test_probe_modes():
    res = {}
    for mode in (nv.PROBE_ZEROS, nv.PROBE_NVFP4_LIKE, nv.PROBE_UNIFORM):
        say("probe_mfma mode", mode)
        tf, ghz = nv.probe_mfma(mode, 2000)
        assert 100.0 < tf <= PEAK_FP16_TFLOPS * 1.02, (mode, tf)
        assert 0.3 < ghz < 3.0, (mode, ghz)
        res[mode] = tf
    # operands that draw less power never run slower
    assert res[nv.PROBE_ZEROS] >= 0.9 * res[nv.PROBE_UNIFORM]
