"""Pins of the MXFP4 oracle (the comparison format: 32-element blocks,
power-of-two E8M0 scale, no tensor scale -- "Pretraining Large Language Models
with NVFP4", summary page, format paragraph) against things other than
itself: a hand-worked example, the defining bound and minimality of the scale
checked in exact rational arithmetic, the page's worst-case statement, float64
brute force, an independently written numpy model, and exact rational GEMM
sums."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), np.asarray(x, np.float32)), "inputs must be bf16-exact"
    return t.view(torch.int16).numpy().view(np.uint16)


def unpack(codes: np.ndarray) -> np.ndarray:
    return model.unpack(codes)


def _value(tok: str) -> float:
    if "*2^" in tok:
        a, b = tok.split("*2^")
        return float(a) * 2.0 ** int(b)
    if tok.startswith("-2^"):
        return -(2.0 ** int(tok[3:]))
    if tok.startswith("2^"):
        return 2.0 ** int(tok[2:])
    return float(tok)


def _golden():
    meta, blocks = {}, []
    with open(os.path.join(GOLDEN, "mxfp4_hand_blocks.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            if "|" not in line:
                k, *v = line.split()
                meta[k] = [int(t) for t in v]
                continue
            pos, e, vals, codes = line.split("|")
            r, b = (int(t) for t in pos.split())
            blocks.append((r, b, int(e), [_value(t) for t in vals.split()],
                           [int(t, 16) for t in codes.split()]))
    return meta, blocks


def test_hand_worked_example():
    meta, blocks = _golden()
    rows, cols = meta["shape"]
    x = np.zeros((rows, cols), np.float32)
    for r, b, _, vals, _ in blocks:
        x[r, 32 * b:32 * b + 32] = vals
    q = oracle.mx_quantize(bf16_bits(x))
    codes = unpack(q.codes)
    for r, b, e, _, expect in blocks:
        assert q.scales[r, b] == e, (r, b, q.scales[r, b])
        assert list(codes[r, 32 * b:32 * b + 32]) == expect, (r, b)


# ------------------------------------------------------------------ the scale
def _amax_samples():
    rng = np.random.default_rng(3)
    vals = [6.0 * 2.0 ** k for k in range(-126, 126)]
    vals += [np.nextafter(np.float32(v), np.float32(np.inf)) for v in vals[::7]]
    vals += [np.nextafter(np.float32(v), np.float32(0)) for v in vals[::7]]
    vals += list((2.0 ** rng.uniform(-149, 127.9, 20000)).astype(np.float32))
    vals += [np.float32(1e-45), np.float32(2.0 ** -126), np.float32(3.3895e38)]
    a = np.array(vals, np.float32)
    return a[np.isfinite(a) & (a > 0)]


def test_e8m0_is_the_smallest_power_of_two_bound():
    """E = 2^(code - 127) satisfies amax <= 6 E, and no smaller power of two
    does unless the exponent is clamped at -127 (exact rationals)."""
    a = _amax_samples()
    codes = oracle.e8m0_encode(a)
    for amax, c in zip(a, codes):
        A = Fraction(float(amax))
        e = int(c) - 127
        assert A <= 6 * Fraction(2) ** e, (amax, c)
        if e > -127:
            assert A > 6 * Fraction(2) ** (e - 1), (amax, c)
    assert oracle.e8m0_encode(np.array([0.0], np.float32))[0] == 0


def test_e8m0_matches_independent_model():
    a = _amax_samples()
    assert np.array_equal(oracle.e8m0_encode(a), model.e8m0_encode(a))


def test_e8m0_decode_is_the_power_of_two():
    for c in range(255):
        assert oracle.e8m0_decode(c) == math.ldexp(1.0, c - 127)


def test_block_max_lands_in_3_to_6():
    """Rounding the exponent up puts every block's largest |v| in (3, 6]."""
    g = torch.Generator().manual_seed(5)
    for std in (1.0, 1e-3, 40.0):
        x = (torch.randn(64, 256, generator=g) * std).to(torch.bfloat16)
        z = x.float().numpy().astype(np.float64)
        q = oracle.mx_quantize(x)
        amax_b = np.abs(z).reshape(64, 8, 32).max(axis=2)
        vmax = amax_b * np.ldexp(1.0, 127 - q.scales.astype(np.int64))
        assert np.all(vmax > 3.0) and np.all(vmax <= 6.0)


def test_worst_case_leaves_4_and_6_unused():
    """A block whose largest |z| sits just above 3 * 2^k gets scale 2^k, so
    |v| <= 3.0234 and the levels 4 and 6 never occur (the page's worst case
    of the power-of-two scale)."""
    rng = np.random.default_rng(7)
    for k in (-20, -1, 0, 3, 40):
        z = rng.uniform(-1, 1, (16, 32)) * 3.0 * 2.0 ** k
        z[:, 0] = 3.0234375 * 2.0 ** k                       # bf16-exact, just above 3 * 2^k
        x = bf16_bits(torch.from_numpy(z.astype(np.float32)).to(torch.bfloat16).float().numpy())
        q = oracle.mx_quantize(x)
        assert np.all(q.scales == 127 + k)
        idx = unpack(q.codes) & 7
        assert not np.any(idx >= 6)


# ------------------------------------------------------------------ encode
def _nearest_even(v: np.ndarray) -> np.ndarray:
    """float64 brute force: nearest of the 8 magnitudes, ties to even index,
    saturating at 6; sign from the sign bit."""
    a = np.minimum(np.abs(v), 6.0)
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    d = np.abs(a[..., None] - mags)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    idx = np.where(even < 99, even, cand.min(axis=-1))
    return (np.signbit(v) * 8 + idx).astype(np.uint8)


def test_rtn_codes_are_nearest_values():
    g = torch.Generator().manual_seed(9)
    x = (torch.randn(48, 512, generator=g) * 3).to(torch.bfloat16)
    x[0, :7] = torch.tensor([0.0, -0.0, 6, -6, 1e-30, -1e30, 0.125], dtype=torch.bfloat16)
    q = oracle.mx_quantize(x)
    z = x.float().numpy().astype(np.float64)
    v = z * np.repeat(np.ldexp(1.0, 127 - q.scales.astype(np.int64)), 32, axis=1)
    assert np.array_equal(unpack(q.codes), _nearest_even(v))


@settings(max_examples=40, deadline=None)
@given(rows=st.integers(1, 6), nb=st.integers(1, 5), seed=st.integers(0, 2**31),
       scale=st.sampled_from([1e-35, 1e-3, 1.0, 7.0, 1e30]), sr=st.booleans())
def test_c_matches_numpy_model(rows, nb, seed, scale, sr):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(rows, 32 * nb, generator=g) * scale).to(torch.bfloat16)
    x[0, 0] = 0.0
    bits = x.view(torch.int16).numpy().view(np.uint16)
    q = oracle.mx_quantize(x, sr_seed=seed if sr else None, stream_id=3)
    codes, sc = model.mx_quantize(bits, sr_seed=seed if sr else None, stream_id=3)
    assert np.array_equal(q.scales, sc)
    assert np.array_equal(unpack(q.codes), codes)


def test_sr_is_unbiased_and_picks_neighbours():
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(2, 64, generator=g)).to(torch.bfloat16)
    z = x.float().numpy().astype(np.float64)
    rtn = oracle.mx_quantize(x)
    acc = np.zeros_like(z)
    n = 4000
    for s in range(n):
        q = oracle.mx_quantize(x, sr_seed=s)
        assert np.array_equal(q.scales, rtn.scales)
        d = oracle.mx_dequantize(q).astype(np.float64)
        E = np.repeat(np.ldexp(1.0, q.scales.astype(np.int64) - 127), 32, axis=1)
        acc += d
        # a grid value, and one of the two neighbours of |z| / E
        vals = np.abs(d) / E
        assert np.all(np.isin(vals, [0, .5, 1, 1.5, 2, 3, 4, 6]))
        grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
        a = np.abs(z) / E
        lo = grid[np.searchsorted(grid, a, side="right") - 1]
        hi = grid[np.minimum(np.searchsorted(grid, a, side="right"), 7)]
        assert np.all((vals == lo) | (vals == hi))
    mean = acc / n
    E = np.repeat(np.ldexp(1.0, rtn.scales.astype(np.int64) - 127), 32, axis=1)
    # each draw has variance <= (gap/2)^2 <= (E)^2 (largest gap 2E): 5 sigma
    assert np.all(np.abs(mean - z) <= 5 * E / np.sqrt(n) + 1e-12)


def test_dequantize_is_the_exact_product():
    g = torch.Generator().manual_seed(2)
    x = (torch.randn(8, 128, generator=g) * 5).to(torch.bfloat16)
    q = oracle.mx_quantize(x)
    d = oracle.mx_dequantize(q)
    expect = E2M1[unpack(q.codes)] * np.repeat(np.ldexp(1.0, q.scales.astype(np.int64) - 127), 32, axis=1)
    assert np.array_equal(d.astype(np.float64), expect)


def test_storage_is_4_25_bits_per_element():
    q = oracle.mx_quantize(torch.zeros(32, 1024, dtype=torch.bfloat16))
    bits = 8 * (q.codes.nbytes + q.scales.nbytes) / (32 * 1024)
    assert bits == 4.25


def test_nvfp4_error_below_mxfp4_on_gaussian_data():
    """The page's claim that smaller blocks and E4M3 scales reduce quantization
    error ("NVFP4 Trains with Precision of 16-Bit ...", micro-block scaling and
    E4M3 sections), on N(0,1) data."""
    g = torch.Generator().manual_seed(0)
    x = torch.randn(256, 1024, generator=g).to(torch.bfloat16)
    z = x.float().numpy().astype(np.float64)
    e_nv = oracle.dequantize(oracle.quantize(x, oracle.ROWWISE)).astype(np.float64) - z
    e_mx = oracle.mx_dequantize(oracle.mx_quantize(x)).astype(np.float64) - z
    assert np.mean(e_nv ** 2) < 0.8 * np.mean(e_mx ** 2)


# ------------------------------------------------------------------ GEMM
def _random_mx(rows, k, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, k, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 3)
    return oracle.mx_quantize(x.to(torch.bfloat16))


def test_gemm_exact_rational_sum():
    a, b = _random_mx(3, 32, 1), _random_mx(4, 32, 2)
    c, t = oracle.mx_gemm(a, b)
    A = unpack(a.codes)
    B = unpack(b.codes)
    for m in range(3):
        for n in range(4):
            s = Fraction(0)
            for k in range(32):
                va = Fraction(float(E2M1[A[m, k]])) * Fraction(2) ** (int(a.scales[m, k // 32]) - 127)
                vb = Fraction(float(E2M1[B[n, k]])) * Fraction(2) ** (int(b.scales[n, k // 32]) - 127)
                s += va * vb
            assert c[m, n] == float(s)


def test_gemm_equals_matmul_of_dequantized():
    a, b = _random_mx(40, 256, 3), _random_mx(24, 256, 4)
    c, t = oracle.mx_gemm(a, b)
    ref = oracle.mx_dequantize(a).astype(np.float64) @ oracle.mx_dequantize(b).astype(np.float64).T
    assert np.all(np.abs(c - ref) <= 1e-12 * t)
    assert np.all(t >= np.abs(c))
    ce, te = oracle.mx_gemm_entries(a, b, np.array([0, 39, 7]), np.array([0, 23, 11]))
    assert np.array_equal(ce, c[[0, 39, 7], [0, 23, 11]])
    assert np.array_equal(te, t[[0, 39, 7], [0, 23, 11]])


def test_gemm_one_hot_selects_an_element():
    a = _random_mx(5, 64, 6)
    x = np.zeros((1, 64), np.float32)
    x[0, 37] = 1.0
    e = oracle.mx_quantize(bf16_bits(x))
    assert e.scales[0, 1] == 125                     # amax 1 <= 6 * 2^-2 -> e = -2 (v = 4)
    c, _ = oracle.mx_gemm(a, e)
    assert np.array_equal(c[:, 0], oracle.mx_dequantize(a)[:, 37].astype(np.float64))


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.mx_quantize(torch.zeros(4, 48, dtype=torch.bfloat16))


def test_decode_exact_is_the_exact_product_wide_scales():
    """Every element, across a range of E8M0 exponents far beyond binary32's
    comfortable range for products (rows scaled by 2^-60 .. 2^60)."""
    g = torch.Generator().manual_seed(8)
    x = torch.randn(64, 128, generator=g) * torch.pow(2.0, torch.arange(64).float() * 2 - 60)[:, None]
    q = oracle.mx_quantize(x.to(torch.bfloat16))
    d = oracle.mx_decode_exact(q)
    expect = E2M1[unpack(q.codes)] * np.repeat(np.ldexp(1.0, q.scales.astype(np.int64) - 127), 32, axis=1)
    assert d.dtype == np.float64 and np.array_equal(d, expect)
    assert q.scales.min() < 100 and q.scales.max() > 160


def test_gemm_f64_k32_equals_exact_rational():
    """One block along K: every float64 sum is exact, so the matmul form
    equals mx_gemm (pinned by the rational test above) exactly."""
    a, b = _random_mx(3, 32, 1), _random_mx(4, 32, 2)
    c, t = oracle.mx_gemm_f64(a, b)
    ce, te = oracle.mx_gemm(a, b)
    assert np.array_equal(c, ce) and np.array_equal(t, te)


def test_gemm_f64_within_float64_bound_of_the_loop():
    """Two float64 summation orders of the same exact products: within
    2 K 2^-53 T of each other."""
    for rows_a, rows_b, k, sa, sb in [(40, 24, 256, 3, 4), (16, 48, 4096, 5, 6)]:
        a, b = _random_mx(rows_a, k, sa), _random_mx(rows_b, k, sb)
        c, t = oracle.mx_gemm_f64(a, b)
        ce, te = oracle.mx_gemm(a, b)
        bound = 2 * k * 2.0 ** -53 * te
        assert np.all(np.abs(c - ce) <= bound) and np.all(np.abs(t - te) <= bound)
