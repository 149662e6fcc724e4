"""The measurement probes on the GPU: the matrix-core probe (sane throughput
and clock for every operand kind, never above the published dense FP16
peak), the plain copy kernel (every byte, nothing past the end) and the clock
stamps (a clock near the one the matrix-core probe reads inside its waves)."""
import pytest
import torch

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


def test_probe_copy_moves_every_byte():
    import bit_microscaled_numerics_amd as nv
    g = torch.Generator(device="cuda").manual_seed(3)
    for n in (16, 4096 * 16 + 48, (1 << 22) + 16 * 5):
        src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
        dst = torch.zeros(n + 64, dtype=torch.uint8, device="cuda")
        nv.probe_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst[:n], src) and not dst[n:].any()


def test_clock_stamps_give_a_plausible_clock():
    """Stamps around a ~50 ms matrix-core run report a clock near the one the
    probe measures inside its own waves, and within the chip's range."""
    import bit_microscaled_numerics_amd as nv
    st = nv.ClockStamps()
    st.before()
    tf, ghz_probe = nv.probe_mfma(nv.PROBE_NVFP4_LIKE, 200000)
    st.after()
    ghz = st.ghz()
    assert 0.5 < ghz < 2.6, ghz
    assert abs(ghz - ghz_probe) < 0.15 * ghz_probe, (ghz, ghz_probe)
