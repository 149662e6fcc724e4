"""CPU check of the near-decision-point inputs (tests/near_points.py) with the
CPU reference: every constructed block gets the intended E4M3 code from the
reference's quantizer, and the reference's scaled values v = z * r of the
rowwise and 2D tensors come within 16 binary32 patterns of every E2M1
midpoint and grid value, below and above (above 6 only by saturation's
neighbourhood, which the construction leaves out), so the GPU test that uses
them exercises the hardware FP4 encode on both sides of every point where
its decision changes."""
import numpy as np

import oracle
import near_points as npz


def _check(tensors, build, mode, blk_rows):
    cov = {}
    rng = np.random.default_rng(1)
    for t in tensors:
        x = build(t, rng)
        q = oracle.quantize(x, mode, amax_given=t.amax)
        assert q.tensor_scale == oracle.tensor_scale(t.amax)
        codes = set(np.unique(q.scales).tolist())
        assert {b.code for b in t.blocks} <= codes
        v = npz.scaled_values(x, t.amax, q.scales, blk_rows)
        for k, n in npz.window_coverage(v).items():
            cov[k] = cov.get(k, 0) + n
    missing = [k for k, n in cov.items() if n == 0 and k != (6.0, 1)]
    assert not missing, missing
    return cov


def test_rowwise_blocks_cover_every_decision_point():
    _check(npz.find(0), lambda t, rng: npz.rowwise_tensor(t, rng), oracle.ROWWISE, 1)


def test_2d_tiles_cover_every_decision_point():
    _check(npz.find(1), lambda t, rng: npz.tiles_2d(t, rng), oracle.TWO_D, 16)
