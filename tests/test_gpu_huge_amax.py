"""Tensors whose RHT amax exceeds 2^125.  The RHT encoders normally fold the
transform's 1/4 into the element scale (y * (r / 4) in place of (y / 4) * r,
the same binary32 while r / 4 is normal); above a tensor amax of 2^125 the
smallest reciprocal's quarter could be subnormal, so every element is
quartered first, as in the plain transform.  Blocks whose sign-flipped values
all equal +c (c = 2e37) transform to 16c in one position, so the tensor amax
after the transform is 4c = 8e37 with no binary32 overflow on the way; the
other blocks are random at a smaller scale, one tile is zero.  Colwise and
rowwise RHT (RTN and SR), the fused rowwise + RHT-transpose kernel and the
RHT amaxes, byte for byte against the CPU reference ("NVFP4 Trains with
Precision of 16-Bit and Speed and Efficiency of 4-Bit", Hadamard-transforms
paragraph)."""
import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
from parity import assert_operand_equal, dev_scalar, f32_bits, say

pytestmark = pytest.mark.gpu

SEED = 7
C = np.float32(2e37)


def _tensor(rng, rows, cols, along_rows: bool) -> torch.Tensor:
    """bf16 [rows][cols]; every third 16-block along the transform axis
    (rows for along_rows, else columns) is c times the sign flips."""
    s = oracle.rht_signs(SEED)
    flips = np.where([(s >> j) & 1 for j in range(16)], -1.0, 1.0).astype(np.float32)
    x = (rng.standard_normal((rows, cols)) * 1e35).astype(np.float32)
    x[:16, :16] = 0.0
    k = 0
    if along_rows:
        for i in range(16, rows, 16):
            for j in range(cols):
                if k % 3 == 0:
                    x[i:i + 16, j] = C * flips
                k += 1
    else:
        for i in range(16, rows):
            for j in range(0, cols, 16):
                if k % 3 == 0:
                    x[i, j:j + 16] = C * flips
                k += 1
    return torch.from_numpy(x).to(torch.bfloat16)


@pytest.mark.parametrize("sr", [None, 93])
def test_huge_amax_colwise_rht(sr):
    rng = np.random.default_rng(11)
    x = _tensor(rng, 64, 96, along_rows=True)
    a_rht = oracle.amax_rht(x, SEED)
    assert a_rht > 2.0 ** 125 and np.isfinite(a_rht), a_rht
    kw = {} if sr is None else {"sr_seed": sr, "stream_id": 4}
    say("huge amax colwise rht", a_rht, sr)
    xd = x.cuda()
    g = nv.rht_quantize(xd, SEED, **kw)
    g_r, g_t = nv.quantize_row_rht(xd, SEED, sr_seed=sr, stream_ids=(4, 5))
    torch.cuda.synchronize()
    assert_operand_equal(g, oracle.quantize(x, oracle.COLWISE, rht_seed=SEED, **kw), "rht col")
    kr = {} if sr is None else {"sr_seed": sr, "stream_id": 4}
    kt = {} if sr is None else {"sr_seed": sr, "stream_id": 5}
    assert_operand_equal(g_r, oracle.quantize(x, oracle.ROWWISE, **kr), "fused row")
    assert_operand_equal(g_t, oracle.quantize(x, oracle.COLWISE, rht_seed=SEED, **kt), "fused rht")


@pytest.mark.parametrize("sr", [None, 94])
def test_huge_amax_rowwise_rht(sr):
    rng = np.random.default_rng(12)
    x = _tensor(rng, 48, 128, along_rows=False)
    kw = {} if sr is None else {"sr_seed": sr, "stream_id": 6}
    o = oracle.quantize(x, oracle.ROWWISE, rht_seed=SEED, **kw)
    assert o.amax > 2.0 ** 125 and np.isfinite(o.amax), o.amax
    say("huge amax rowwise rht", o.amax, sr)
    g = nv.rht_quantize(x.cuda(), SEED, axis=nv.NVFP4_ROWWISE, **kw)
    torch.cuda.synchronize()
    assert_operand_equal(g, o, "rht row")


def test_huge_amax_rht_amaxes():
    """The amax passes take the 1/4 on the maximum: the same binary32."""
    rng = np.random.default_rng(13)
    xc = _tensor(rng, 64, 96, along_rows=True)
    xr = _tensor(rng, 48, 128, along_rows=False)
    say("huge amax rht amaxes")
    _, a_col = nv.amax_both(xc.cuda(), SEED)
    a_row = nv.amax_rht(xr.cuda(), SEED, axis=nv.NVFP4_ROWWISE)
    torch.cuda.synchronize()
    assert f32_bits(dev_scalar(a_col)) == f32_bits(oracle.amax_rht(xc, SEED))
    o = oracle.quantize(xr, oracle.ROWWISE, rht_seed=SEED)
    assert f32_bits(dev_scalar(a_row)) == f32_bits(o.amax)
