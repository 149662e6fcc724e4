"""The hardware FP4 encode inside the quantizer kernels, fed scaled values
v = z * r within 16 binary32 patterns of every E2M1 midpoint and grid value
(tests/near_points.py: tensor amaxes, block codes and bf16 elements solved
so that the non-power-of-two element scales put v there), through the C ABI:
rowwise, colwise (fed the transpose, so its blocks are the same), 2D tiles
and the fused rowwise + RHT-transpose kernel; round-to-nearest-even and
stochastic rounding; codes and scales byte for byte against the CPU
reference.  (MXFP4 is not among them: its power-of-two scales make v a
scaled bf16 value, which the all-values test already covers.)  Sources:
"Pretraining Large Language Models with NVFP4", format paragraph; "NVFP4
Trains with Precision of 16-Bit and Speed and Efficiency of 4-Bit",
stochastic rounding."""
import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
import near_points as npz
from parity import assert_operand_equal, say

pytestmark = pytest.mark.gpu

SR = [None, 0x0DDB1A5E5BAD5EED]


def _bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def _amax(a: float) -> torch.Tensor:
    return torch.tensor([a], dtype=torch.float32, device="cuda")


def _kw(sr, stream_id=0):
    return {} if sr is None else {"sr_seed": sr, "stream_id": stream_id}


@pytest.mark.parametrize("sr", SR)
def test_rowwise_and_colwise(sr):
    rng = np.random.default_rng(2)
    for i, t in enumerate(npz.find(0)):
        x = _bf16(npz.rowwise_tensor(t, rng))
        say("near points rowwise/colwise", i, tuple(x.shape), t.amax, sr)
        g = nv.quantize_1d(x.cuda(), amax=_amax(t.amax), **_kw(sr, 2))
        xt = x.t().contiguous()
        gc = nv.quantize_1d(xt.cuda(), nv.NVFP4_COLWISE, amax=_amax(t.amax), **_kw(sr, 2))
        torch.cuda.synchronize()
        o = oracle.quantize(x, oracle.ROWWISE, amax_given=t.amax, **_kw(sr, 2))
        assert_operand_equal(g, o, f"row {i} sr={sr}")
        oc = oracle.quantize(xt, oracle.COLWISE, amax_given=t.amax, **_kw(sr, 2))
        assert_operand_equal(gc, oc, f"col {i} sr={sr}")


@pytest.mark.parametrize("sr", SR)
def test_2d(sr):
    rng = np.random.default_rng(3)
    for i, t in enumerate(npz.find(1)):
        x = _bf16(npz.tiles_2d(t, rng))
        say("near points 2d", i, tuple(x.shape), t.amax, sr)
        g = nv.quantize_2d(x.cuda(), amax=_amax(t.amax), **_kw(sr, 4))
        torch.cuda.synchronize()
        o = oracle.quantize(x, oracle.TWO_D, amax_given=t.amax, with_codes_t=True, **_kw(sr, 4))
        assert_operand_equal(g, o, f"2d {i} sr={sr}")


@pytest.mark.parametrize("sr", SR)
def test_fused_rowwise_and_rht(sr):
    rng = np.random.default_rng(4)
    for i, t in enumerate(npz.find(2)):
        x = _bf16(npz.rowwise_tensor(t, rng, cols_blocks=8))
        R, C = x.shape
        a_rht = oracle.amax_rht(x, 55)
        say("near points fused", i, (R, C), t.amax, a_rht, sr)
        e = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")  # noqa: E731
        f = lambda: torch.empty(1, dtype=torch.float32, device="cuda")    # noqa: E731
        gr = nv.NVFP4Tensor(e(R, C // 2), e(R, C // 16), f(), _amax(t.amax), R, C, 1, C // 16, 1)
        gt = nv.NVFP4Tensor(e(C, R // 2), e(C, R // 16), f(), _amax(a_rht), C, R, 1, R // 16, 1)
        nv.nvfp4_quantize_row_rht(x.cuda(), 55, sr is not None, sr or 0, 6, 7, gr.amax, gt.amax,
                                  gr.codes, gr.scales, gr.tensor_scale, gt.codes, gt.scales,
                                  gt.tensor_scale)
        torch.cuda.synchronize()
        assert_operand_equal(gr, oracle.quantize(x, oracle.ROWWISE, amax_given=t.amax,
                                                 **_kw(sr, 6)), f"fused row {i} sr={sr}")
        assert_operand_equal(gt, oracle.quantize(x, oracle.COLWISE, rht_seed=55,
                                                 amax_given=a_rht, **_kw(sr, 7)),
                             f"fused rht {i} sr={sr}")
