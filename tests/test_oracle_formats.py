"""Pins of the oracle's number formats and random bits against things other
than itself: published Philox known answers, torch's float8_e4m3fn cast, a
float64 brute-force nearest search, exact counting over all 2^16 random
values, and the E2M1 value set printed on the pages.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_SET = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ------------------------------------------------------------------ Philox
def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(t, 16) for t in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_philox_known_answers(ctr, key, expect):
    assert oracle.philox4x32_10(ctr, key) == expect
    got = model.philox(np.array([ctr], np.uint64), key[0], key[1])[0]
    assert [int(v) for v in got] == expect


def test_sr_bits_eight_elements_per_call():
    """Eight consecutive operand indices share one Philox call (counter
    n/8, stream id in word 2); each takes a distinct 16-bit half."""
    seed, sid = 0x1234_5678_9ABC_DEF0, 7
    for g in [0, 1, 12345, (1 << 32) + 5]:
        words = oracle.philox4x32_10([g & 0xFFFFFFFF, g >> 32, sid, 0],
                                     [seed & 0xFFFFFFFF, seed >> 32])
        halves = []
        for w in words:
            halves += [w & 0xFFFF, w >> 16]
        assert list(oracle.sr_bits(seed, sid, 8 * g, 8)) == halves


def test_sr_bits_model_agrees_and_streams_differ():
    rng = np.random.default_rng(0)
    n = rng.integers(0, 1 << 40, size=4096, dtype=np.uint64)
    for seed, sid in [(1, 0), (1, 1), (2**63 + 3, 5)]:
        ref = np.array([oracle.sr_bits(seed, sid, int(v), 1)[0] for v in n[:256]])
        assert np.array_equal(model.sr_bits(seed, sid, n[:256]), ref)
    a = oracle.sr_bits(1, 0, 0, 1 << 16)
    b = oracle.sr_bits(1, 1, 0, 1 << 16)
    c = oracle.sr_bits(2, 0, 0, 1 << 16)
    assert np.mean(a == b) < 0.001 and np.mean(a == c) < 0.001


def test_sr_bits_uniform_and_uncorrelated():
    u = oracle.sr_bits(1, 0, 0, 1 << 20).astype(np.int64)
    # chi-square on the top byte: 255 dof, mean 255, sd ~22.6
    counts = np.bincount(u >> 8, minlength=256)
    expect = u.size / 256
    chi2 = float(np.sum((counts - expect) ** 2 / expect))
    assert 255 - 6 * 22.6 < chi2 < 255 + 6 * 22.6
    # every bit is balanced to ~6 sigma
    for b in range(16):
        frac = np.mean((u >> b) & 1)
        assert abs(frac - 0.5) < 6 * 0.5 / math.sqrt(u.size)
    # neighbours (same call and across calls) are uncorrelated
    x = u.astype(np.float64) - 32767.5
    for lag in (1, 2, 7, 8):
        r = np.mean(x[:-lag] * x[lag:]) / np.mean(x * x)
        assert abs(r) < 6 / math.sqrt(u.size)


def test_rht_signs_match_model():
    for s in [0, 1, 42, 2**64 - 1]:
        assert oracle.rht_signs(s) == model.rht_signs(s)
    assert oracle.rht_signs(1) != oracle.rht_signs(2)


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_torch():
    codes = torch.arange(0, 127, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(127)], np.float32)
    assert np.array_equal(got, ref)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.array_equal(model.e4m3_value(np.arange(127)), ref)


def test_e4m3_encode_matches_torch_exhaustive():
    """Every binary32 in [0, 464]: the oracle equals torch's RNE cast."""
    top = np.float32(464.0).view(np.uint32)
    chunk = 1 << 24
    start = 0
    while start <= top:
        stop = min(start + chunk, int(top) + 1)
        bits = np.arange(start, stop, dtype=np.uint32)
        x = bits.view(np.float32)
        got = oracle.e4m3_encode(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"first mismatch at x={x[bad[0]]!r}: {got[bad[0]]} vs {ref[bad[0]]}"
        start = stop


def test_e4m3_encode_saturates_and_model_agrees():
    x = np.array([448.0, 464.0, 465.0, 500.0, 1e6, 3.4e38, np.inf], np.float32)
    assert np.all(oracle.e4m3_encode(x[:-1]) == 0x7E)
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(0, 500, 100000), 2.0 ** rng.uniform(-14, 9, 100000),
                        [0.0, 2.0 ** -10, 1.5 * 2.0 ** -10, 2.0 ** -9]]).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(y), model.e4m3_encode(y))
    assert oracle.e4m3_encode(np.float32([2.0 ** -10]))[0] == 0       # tie to even (0)
    assert oracle.e4m3_encode(np.float32([1.5 * 2.0 ** -10]))[0] == 1  # tie to even (2^-9)


# ------------------------------------------------------------------ E2M1
def test_e2m1_codes_decode_to_the_printed_value_set():
    """The 16 codes are 0, +-0.5 ... +-6: the value set of the element format."""
    vals = [oracle.e2m1_decode(c) for c in range(16)]
    assert vals[:8] == E2M1_SET
    assert [-v for v in vals[8:]] == E2M1_SET
    assert math.copysign(1.0, vals[8]) == -1.0          # code 8 is -0
    assert len(set(abs(v) for v in vals)) == 8 and len(vals) == 16


def _nearest_even_f64(a):
    """float64 brute force: argmin |a - g| over the grid, ties to even index,
    saturate above 6."""
    g = np.array(E2M1_SET)
    d = np.abs(a[:, None].astype(np.float64) - g[None, :])
    best = np.argmin(d, axis=1)                     # first (lower) index on a tie
    tie_up = np.zeros_like(best, dtype=bool)
    nxt = np.minimum(best + 1, 7)
    tie = d[np.arange(a.size), nxt] == d[np.arange(a.size), best]
    tie_up = tie & (best % 2 == 1) & (nxt != best)
    return np.where(tie_up, nxt, best)


def test_e2m1_rtn_bruteforce_sampled_and_near_midpoints():
    hi = np.float32(8.0).view(np.uint32)
    bits = np.arange(0, int(hi), 401, dtype=np.uint32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-2000, 2001)[None, :]).ravel()
    bits = np.concatenate([bits, near.astype(np.uint32)])
    a = bits.view(np.float32)
    for lo in range(0, a.size, 1 << 22):
        blk = a[lo:lo + (1 << 22)]
        got = oracle.e2m1_rtn(blk)
        ref = _nearest_even_f64(blk)
        assert np.array_equal(got, ref.astype(np.uint8))
        assert np.array_equal(oracle.e2m1_rtn(-blk), ref.astype(np.uint8) | 8)
        assert np.array_equal(model.e2m1_rtn(blk), got)


def test_e2m1_rtn_ties_and_saturation():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert list(oracle.e2m1_rtn(ties)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(oracle.e2m1_rtn(np.float32([6.0, 7.0, 1e30, -9.0]))) == [7, 7, 7, 15]
    assert list(oracle.e2m1_rtn(np.float32([0.0, -0.0]))) == [0, 8]


def test_e2m1_sr_exact_counts_over_all_random_values():
    """For each v, the number of u16 in [0, 2^16) that round up is exactly
    ceil(p * 2^16) with p = (a - lo)/(hi - lo) computed exactly; so the mean
    over the random values is within gap * 2^-16 of a (unbiased)."""
    rng = np.random.default_rng(2)
    vs = np.concatenate([rng.uniform(0, 6, 300), rng.uniform(0, 0.5, 50),
                         np.array([0.1, 0.25, 0.3333, 2.9999, 4.5, 5.999])]).astype(np.float32)
    u = np.arange(1 << 16, dtype=np.uint16)
    g = np.array(E2M1_SET)
    for v in vs:
        codes = oracle.e2m1_sr(np.full(1 << 16, v, np.float32), u)
        a = float(v)
        lo = int(np.searchsorted(g, a, side="right") - 1)
        if g[lo] == a:
            assert np.all(codes == lo)
            continue
        p = (a - g[lo]) / (g[lo + 1] - g[lo])
        ups = int(np.sum(codes == lo + 1))
        assert ups + int(np.sum(codes == lo)) == 1 << 16
        assert ups == math.ceil(p * 65536)
        mean = float(np.mean(g[codes]))
        assert abs(mean - a) <= (g[lo + 1] - g[lo]) * 2.0 ** -16 + 1e-15
        assert np.array_equal(model.e2m1_sr(np.full(1 << 16, v, np.float32), u), codes)


def test_e2m1_sr_grid_points_fixed_sign_and_saturation():
    u = np.arange(1 << 16, dtype=np.uint16)
    for i, gv in enumerate(E2M1_SET):
        assert np.all(oracle.e2m1_sr(np.full(1 << 16, gv, np.float32), u) == i)
        assert np.all(oracle.e2m1_sr(np.full(1 << 16, -gv, np.float32), u) == (8 | i))
    assert np.all(oracle.e2m1_sr(np.full(1 << 16, 9.0, np.float32), u) == 7)


def test_e2m1_sr_unbiased_over_seeds():
    """Mean over many seeds of the rounded value approaches the input."""
    v = np.float32(0.3)
    seeds = np.arange(1, 10001)
    u = np.array([oracle.sr_bits(int(s), 0, 5, 1)[0] for s in seeds], np.uint16)
    codes = oracle.e2m1_sr(np.full(seeds.size, v, np.float32), u)
    vals = np.array(E2M1_SET)[codes & 7]
    p = 0.3 / 0.5
    sigma = 0.5 * math.sqrt(p * (1 - p) / seeds.size)
    assert abs(vals.mean() - 0.3) < 4 * sigma + 0.5 * 2 ** -16


def test_e2m1_rtn_exhaustive_step_function():
    """Every binary32 in [0, 8] (1.09e9 values, in chunks): the RTN code is a
    non-decreasing step function of the value that changes exactly seven
    times, each time by one, at the midpoints between grid values: the upper
    code takes the midpoint itself where its index is even (0.75, 1.75, 3.5)
    and starts one ulp above where it is odd (0.25, 1.25, 2.5, 5).  Codes of
    values in (6, 8] stay at 7."""
    end = int(np.float32(8.0).view(np.uint32))
    step = 1 << 24
    idx = np.arange(step, dtype=np.uint32)
    buf = np.empty(step, np.uint32)
    changes = []
    prev = None
    for lo in range(0, end + 1, step):
        n = min(step, end + 1 - lo)
        bits = np.add(idx[:n], np.uint32(lo), out=buf[:n])
        codes = oracle.e2m1_rtn(bits.view(np.float32))
        if prev is not None:
            assert codes[0] >= prev
            if codes[0] != prev:
                changes.append((lo, int(prev), int(codes[0])))
        up = codes[1:] != codes[:-1]
        if up.any():
            for i in np.nonzero(up)[0]:
                assert codes[i + 1] == codes[i] + 1
                changes.append((lo + int(i) + 1, int(codes[i]), int(codes[i + 1])))
        prev = codes[-1]
    f = lambda x: int(np.float32(x).view(np.uint32))   # noqa: E731
    expect = [(f(0.25) + 1, 0, 1), (f(0.75), 1, 2), (f(1.25) + 1, 2, 3), (f(1.75), 3, 4),
              (f(2.5) + 1, 4, 5), (f(3.5), 5, 6), (f(5.0) + 1, 6, 7)]
    assert changes == expect
