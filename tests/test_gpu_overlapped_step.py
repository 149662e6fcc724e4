"""The benchmark step with its independent quantization chains on a second
stream (bench.Step.run_overlapped) produces exactly the bytes of the serial
step (bench.Step.run): every quantized operand, Y, dX and dW, bit for bit,
on three overlapped steps in a row."""
import numpy as np
import pytest
import torch

import bench
from bit_microscaled_numerics_amd import inputs
from parity import say

pytestmark = pytest.mark.gpu


def _outputs(step):
    out = []
    for q in (step.qx, step.qw, step.qdy, step.qdy_t, step.qx_t):
        for t in (q.codes, q.scales, q.tensor_scale, q.amax, q.codes_t, q.scales_t):
            if t is not None:
                out.append(t)
    return out + [step.y, step.dx, step.dw]


@pytest.mark.parametrize("shape", [(512, 256, 1024), (1024, 512, 2048)])
def test_overlapped_step_matches_serial(shape):
    T, H, F = shape
    wl = inputs.ffn_down(3, T, H, F)
    dev = torch.device("cuda")
    step = bench.Step(*(wl.tensors[k].to(dev) for k in ("X", "W", "dY")))
    say("overlapped step", shape)
    step.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in _outputs(step)]
    for _ in range(3):
        for t in _outputs(step):
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        step.run_overlapped()
        torch.cuda.synchronize()
        for a, b in zip(_outputs(step), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert np.isfinite(ref[-1].cpu().numpy()).all()
