"""Block scales whose quotient amax_b / (6 s_t) lies exactly on a point where
the E4M3 code changes: the midpoint between two neighbouring E4M3 values,
where round-to-nearest-even must pick the even code.

Construction: the tensor amax is 784 * 2^k, so s_t = fl(amax / 2688) and
t6 = fl(6 s_t) = 1.75 * 2^k exactly; every 16-element block (along the rows)
has max |x| = b = 1.75 * m * 2^k for an E4M3 midpoint m (126 of the 127
midpoints give a b that bf16 holds exactly: m has at most 5 significant bits).
The correctly rounded quotient b / t6 is then m itself, a tie.  A block-scale
step that replaced the division by a multiply with fl(1/t6) would land one ulp
off the tie on 78 of the 126 and round it the wrong way; the HIP kernels
detect quotients that close to a rounding point and divide.  The E4M3
encoding and the tensor scale follow "NVFP4 Trains with Precision of 16-Bit
and Speed and Efficiency of 4-Bit" (E4M3 scale factors) and "Pretraining
Large Language Models with NVFP4" (format paragraph: FP32 tensor scale, E4M3
scale per 16 elements)."""
import numpy as np
import pytest
import torch

import oracle


def e4m3_values() -> np.ndarray:
    """Every finite non-negative E4M3FN value (bias 7, max 448), ascending."""
    sub = [j * 2.0 ** -9 for j in range(8)]
    nrm = [(1 + i / 8) * 2.0 ** e for e in range(-6, 9) for i in range(8)]
    return np.array(sorted(set(sub + [v for v in nrm if v <= 448.0])))


def midpoints() -> np.ndarray:
    v = e4m3_values()
    return (v[:-1] + v[1:]) / 2


def tie_maxima(k: int) -> np.ndarray:
    """Block maxima 1.75 * m * 2^k over the E4M3 midpoints m, where bf16 holds them exactly."""
    b = 1.75 * midpoints() * 2.0 ** k
    exact = torch.from_numpy(b).to(torch.bfloat16).double().numpy() == b
    return b[exact]


def tie_tensor(rows: int, cols: int, k: int, seed: int) -> tuple[torch.Tensor, np.ndarray]:
    """bf16 [rows][cols] and the block maxima it was built with ([rows][cols/16])."""
    maxima = tie_maxima(k)
    rng = np.random.default_rng(seed)
    nb = cols // 16
    x = np.empty((rows, cols), np.float64)
    bmax = np.empty((rows, nb), np.float64)
    for r in range(rows):
        for j in range(nb):
            b = maxima[(r * nb + j) % len(maxima)]
            blk = rng.uniform(-0.98, 0.98, 16) * b
            blk[rng.integers(16)] = b * rng.choice([-1.0, 1.0])
            x[r, 16 * j:16 * j + 16] = blk
            bmax[r, j] = b
    x[0, 0] = 784.0 * 2.0 ** k           # the tensor amax (block (0, 0) loses its tie)
    bmax[0, 0] = x[0, 0]
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16), bmax


@pytest.mark.parametrize("k", [0, -12, 9])
def test_tie_construction(k):
    """The inputs do what the GPU test below needs (numpy float32 arithmetic,
    independent of both implementations), and the oracle rounds every tie to
    the even E4M3 code."""
    x, bmax = tie_tensor(64, 256, k, seed=k + 100)
    xf = x.float().numpy()
    blocks = np.abs(xf.reshape(64, 16, 16)).max(axis=2)
    assert np.array_equal(blocks.astype(np.float64), bmax)       # maxima exact in bf16
    assert len(tie_maxima(k)) == 126
    amax = np.float32(784.0 * 2.0 ** k)
    s_t = amax / np.float32(2688.0)
    t6 = np.float32(6.0) * s_t
    assert t6 == np.float32(1.75 * 2.0 ** k)
    q = blocks / t6                                                # float32 division, RNE
    mids = midpoints()
    on_tie = np.isin(q.astype(np.float64), mids)
    assert on_tie.sum() == on_tie.size - 1                         # all but block (0, 0)
    q_mul = blocks * (np.float32(1.0) / t6)
    assert np.count_nonzero((q_mul != q) & on_tie) >= 64 * 16 // 2   # a multiply misses the tie
    o = oracle.quantize(x, oracle.ROWWISE)
    codes = o.scales.astype(np.int64)
    vals = e4m3_values()
    for r, j in zip(*np.nonzero(on_tie)):
        lo = vals[np.searchsorted(vals, q[r, j]) - 1]
        hi = vals[np.searchsorted(vals, q[r, j])]
        c = codes[r, j]
        assert c % 2 == 0, (r, j, q[r, j], c)
        assert oracle.e4m3_decode(int(c)) in (lo, hi)


@pytest.mark.gpu
@pytest.mark.parametrize("k", [0, -12, 9])
def test_tie_scales_match_oracle(k):
    import bit_microscaled_numerics_amd as nv
    from parity import assert_operand_equal, say

    x, _ = tie_tensor(64, 256, k, seed=k + 100)
    xd = x.cuda()
    xt = x.t().contiguous()
    say("scale ties", k)
    g_row = nv.quantize_1d(xd)
    g_sr = nv.quantize_1d(xd, sr_seed=17, stream_id=2)
    g_col = nv.quantize_1d(xt.cuda(), nv.NVFP4_COLWISE)
    g_2d = nv.quantize_2d(xd)
    g_fr, g_ft = nv.quantize_row_rht(xd, 99)
    torch.cuda.synchronize()
    assert_operand_equal(g_row, oracle.quantize(x, oracle.ROWWISE), f"ties row k={k}")
    assert_operand_equal(g_sr, oracle.quantize(x, oracle.ROWWISE, sr_seed=17, stream_id=2),
                         f"ties row SR k={k}")
    assert_operand_equal(g_col, oracle.quantize(xt, oracle.COLWISE), f"ties col k={k}")
    assert_operand_equal(g_2d, oracle.quantize(x, oracle.TWO_D, with_codes_t=True),
                         f"ties 2d k={k}")
    assert_operand_equal(g_fr, oracle.quantize(x, oracle.ROWWISE), f"ties fused row k={k}")
    assert_operand_equal(g_ft, oracle.quantize(x, oracle.COLWISE, rht_seed=99),
                         f"ties fused rht k={k}")
