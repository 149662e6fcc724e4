"""Every bf16 value in [-6, 6] through the E2M1 decision, RTN and SR.

The tensor amax is 2688 = 6 * 448, so the FP32 tensor scale is exactly 1;
every other 16-element block holds 6.0 as its largest magnitude, so its E4M3
scale is exactly 1 and the element scale 1/(E * s_t) is 1: the encoder sees
the bf16 inputs themselves.  The other 15 elements of those blocks run
through all 16577 non-negative bf16 values up to 6 and their negatives
(every grid point and midpoint of the element format, the binade edges, the
subnormals, signed zeros).  Codes and scales must equal the oracle's byte for
byte: rowwise NVFP4 with round-to-nearest-even and with stochastic rounding
(the E2M1 value set and its scaling: "Pretraining Large Language Models with
NVFP4", format paragraph; the rounding modes: "NVFP4 Trains with Precision of
16-Bit and Speed and Efficiency of 4-Bit", stochastic rounding), and the
MXFP4 comparison format, whose power-of-two scale for a block maximum of 6 is
also 1."""
import numpy as np
import pytest
import torch

import oracle
from parity import assert_operand_equal, say

ROWS, COLS = 144, 256     # 2304 blocks of 16


def all_values_tensor() -> torch.Tensor:
    pos = np.arange(0, 0x40C0 + 1, dtype=np.uint32)          # bf16 bit patterns 0 .. 6.0
    vals = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    x = np.zeros((ROWS * COLS // 16, 16), np.uint16)
    x[:, 0] = 0x40C0                                          # 6.0: every block's max
    flat = x[:, 1:].reshape(-1)
    flat[:vals.size] = vals
    flat[vals.size:] = vals[:flat.size - vals.size]
    x[:, 1:] = flat.reshape(-1, 15)
    x = x.reshape(ROWS, COLS)
    x[0, 0] = np.uint16(np.float32(2688.0).view(np.uint32) >> 16)   # the tensor amax
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)


def test_scales_are_one():
    """CPU check of the construction with the oracle: every non-negative bf16
    value up to 6 and its negative occur, the tensor scale is 1 and every
    block but the first has E4M3 scale code 0x38 (1.0); MXFP4 scales are 127
    (2^0) but the first block's."""
    x = all_values_tensor()
    u = x.view(torch.int16).numpy().view(np.uint16)
    assert np.unique(u).size == 2 * (0x40C0 + 1) + 1          # + the amax element
    o = oracle.quantize(x, oracle.ROWWISE)
    assert o.tensor_scale == 1.0
    sc = o.scales.reshape(-1)
    assert sc[0] == 0x7E and np.all(sc[1:] == 0x38)
    m = oracle.mx_quantize(x).scales.reshape(-1)
    assert m[0] != 127 and np.all(m[1:] == 127)


@pytest.mark.gpu
@pytest.mark.parametrize("sr", [False, True])
def test_nvfp4_rowwise_all_values(sr):
    import bit_microscaled_numerics_amd as nv
    x = all_values_tensor()
    kw = {"sr_seed": 0x5EED_0000_0042, "stream_id": 5} if sr else {}
    say("all bf16 values, nvfp4 rowwise", sr)
    g = nv.quantize_1d(x.cuda(), **kw)
    torch.cuda.synchronize()
    assert_operand_equal(g, oracle.quantize(x, oracle.ROWWISE, **kw), f"all values sr={sr}")


@pytest.mark.gpu
@pytest.mark.parametrize("sr", [False, True])
def test_nvfp4_colwise_2d_and_fused_all_values(sr):
    """The same values through the transpose kernel (fed x^T, so its column
    blocks are x's row blocks), the 2D kernel (every 16x16 tile but the first
    also has maximum 6) and the fused rowwise + RHT kernel."""
    import bit_microscaled_numerics_amd as nv
    x = all_values_tensor()
    xt = x.t().contiguous()
    kw = {"sr_seed": 0x5EED_0000_0043, "stream_id": 6} if sr else {}
    say("all bf16 values, nvfp4 colwise / 2d / fused", sr)
    g_col = nv.quantize_1d(xt.cuda(), nv.NVFP4_COLWISE, **kw)
    g_2d = nv.quantize_2d(x.cuda(), **kw)
    g_r, g_t = nv.quantize_row_rht(x.cuda(), 77, sr_seed=kw.get("sr_seed"), stream_ids=(6, 7))
    torch.cuda.synchronize()
    assert_operand_equal(g_col, oracle.quantize(xt, oracle.COLWISE, **kw), f"col sr={sr}")
    assert_operand_equal(g_2d, oracle.quantize(x, oracle.TWO_D, with_codes_t=True, **kw),
                         f"2d sr={sr}")
    kr = {"sr_seed": kw["sr_seed"], "stream_id": 6} if sr else {}
    kt = {"sr_seed": kw["sr_seed"], "stream_id": 7} if sr else {}
    assert_operand_equal(g_r, oracle.quantize(x, oracle.ROWWISE, **kr), f"fused row sr={sr}")
    assert_operand_equal(g_t, oracle.quantize(x, oracle.COLWISE, rht_seed=77, **kt),
                         f"fused rht sr={sr}")


@pytest.mark.gpu
@pytest.mark.parametrize("sr", [False, True])
def test_mxfp4_all_values(sr):
    import bit_microscaled_numerics_amd as nv
    x = all_values_tensor()
    kw = {"sr_seed": 99, "stream_id": 2} if sr else {}
    say("all bf16 values, mxfp4", sr)
    g = nv.mx_quantize(x.cuda(), **kw)
    torch.cuda.synchronize()
    o = oracle.mx_quantize(x, **kw)
    assert np.array_equal(g.codes.cpu().numpy(), o.codes)
    assert np.array_equal(g.scales.cpu().numpy(), o.scales)
