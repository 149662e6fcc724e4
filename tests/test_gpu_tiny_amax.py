"""Tensors whose amax is so small (about 1e-36) that 1/(6 s_t) overflows
binary32: the kernels' reciprocal-multiply shortcut for the block-scale code
would give inf (NaN for an all-zero block), so every block must take the
correctly rounded division amax_b / (6 s_t) instead.  The block maxima stay
within a factor 4 of the tensor amax, so every non-zero block's element
scale 1/(E s_t) is finite and the CPU reference's codes are well defined;
one 16x16 tile is all zero.  Rowwise (RTN and SR), colwise, 2D, RHT
transpose and the fused rowwise + RHT kernel, amax computed and given, byte
for byte against the reference ("Pretraining Large Language Models with
NVFP4", format paragraph: FP32 tensor scale, E4M3 block scale)."""
import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
from parity import assert_operand_equal, say

pytestmark = pytest.mark.gpu


def _tiles(rng, R, C, mags) -> torch.Tensor:
    """Per 16x16 tile one magnitude m from `mags` (0 for the zero tile): every
    row and every column of the tile holds +-m once, the rest smaller."""
    x = np.zeros((R, C), np.float32)
    t = 0
    for i in range(0, R, 16):
        for j in range(0, C, 16):
            m = mags[t % len(mags)]
            t += 1
            blk = rng.choice(np.float32([0.0, 0.25, 0.5, 0.9]), (16, 16)) * m
            blk[np.arange(16), rng.permutation(16)] = m
            x[i:i + 16, j:j + 16] = blk * rng.choice(np.float32([-1, 1]), (16, 16))
    return torch.from_numpy(x).to(torch.bfloat16)


def _check_divide_path(amax: float):
    s_t = np.float32(oracle.tensor_scale(amax))
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(1.0) / (np.float32(6.0) * s_t)), amax


@pytest.mark.parametrize("sr", [None, 91])
def test_tiny_amax_plain_layouts(sr):
    rng = np.random.default_rng(7)
    x = _tiles(rng, 64, 256, [1.0e-36, 0.0, 0.7e-36, 0.5e-36, 0.3e-36])
    amax = oracle.amax(x)
    _check_divide_path(amax)
    kw = {} if sr is None else {"sr_seed": sr, "stream_id": 1}
    say("tiny amax rowwise/colwise/2d", amax, sr)
    xd = x.cuda()
    g_row = nv.quantize_1d(xd, **kw)
    g_col = nv.quantize_1d(xd, nv.NVFP4_COLWISE, **kw)
    g_2d = nv.quantize_2d(xd, **kw)
    g_given = nv.quantize_1d(xd, amax=torch.tensor([amax], device="cuda"), **kw)
    torch.cuda.synchronize()
    o_row = oracle.quantize(x, oracle.ROWWISE, **kw)
    assert_operand_equal(g_row, o_row, "row")
    assert_operand_equal(g_given, o_row, "row, amax given")
    assert_operand_equal(g_col, oracle.quantize(x, oracle.COLWISE, **kw), "col")
    assert_operand_equal(g_2d, oracle.quantize(x, oracle.TWO_D, with_codes_t=True, **kw), "2d")


@pytest.mark.parametrize("sr", [None, 92])
def test_tiny_amax_rht(sr):
    """All elements +-c (one zero tile): every 16-point transform of them has
    its largest magnitude in [c, 4c], so block maxima stay within a factor 4
    of the amax after the transform too."""
    rng = np.random.default_rng(8)
    x = _tiles(rng, 64, 128, [2.5e-37, 2.5e-37, 0.0, 2.5e-37])
    xf = x.float()
    x = torch.where(xf == 0, xf, torch.sign(xf) * 2.5e-37).to(torch.bfloat16)
    x[16:32, 32:48] = 0
    a_rht = oracle.amax_rht(x, 5)
    _check_divide_path(a_rht)
    kw = {} if sr is None else {"sr_seed": sr, "stream_id": 2}
    say("tiny amax rht", a_rht, sr)
    xd = x.cuda()
    g_rht = nv.rht_quantize(xd, 5, **kw)
    g_r, g_t = nv.quantize_row_rht(xd, 5, sr_seed=sr, stream_ids=(2, 3))
    torch.cuda.synchronize()
    assert_operand_equal(g_rht, oracle.quantize(x, oracle.COLWISE, rht_seed=5, **kw), "rht")
    kr = {} if sr is None else {"sr_seed": sr, "stream_id": 2}
    kt = {} if sr is None else {"sr_seed": sr, "stream_id": 3}
    assert_operand_equal(g_r, oracle.quantize(x, oracle.ROWWISE, **kr), "fused row")
    assert_operand_equal(g_t, oracle.quantize(x, oracle.COLWISE, rht_seed=5, **kt), "fused rht")
