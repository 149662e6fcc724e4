"""Pins of the oracle's 16-point random Hadamard transform: the Sylvester
matrix from scipy, orthogonality (the transform is transparent to the GEMM),
its inverse, and outlier spreading.  CPU only."""
import numpy as np
import scipy.linalg

import oracle
from oracle import model

H16 = scipy.linalg.hadamard(16).astype(np.float64)


def _signs_vec(s):
    return np.array([-1.0 if (s >> j) & 1 else 1.0 for j in range(16)])


def test_butterfly_is_quarter_sylvester_hadamard_times_signs():
    assert np.array_equal(H16 @ H16.T, 16 * np.eye(16))
    for s in [0, 0xFFFF, 0xA5C3, oracle.rht_signs(1)]:
        D = _signs_vec(s)
        for j in range(16):
            e = np.zeros(16, np.float32)
            e[j] = 1.0
            got = oracle.rht16(e, s).astype(np.float64)
            assert np.array_equal(got, 0.25 * H16[:, j] * D[j])   # exact: +-1/4 entries


def test_rht_matches_float64_matrix_product_within_rounding():
    rng = np.random.default_rng(3)
    for _ in range(200):
        x = rng.standard_t(3, 16).astype(np.float32)
        s = int(rng.integers(0, 1 << 16))
        ref = 0.25 * H16 @ (_signs_vec(s) * x.astype(np.float64))
        got = oracle.rht16(x, s).astype(np.float64)
        # 4 levels of float32 adds: each level adds <= 2^-24 relative of the partial sums
        bound = 0.25 * 4 * 2.0 ** -24 * np.sum(np.abs(x)) * 2
        assert np.max(np.abs(got - ref)) <= bound
        assert np.array_equal(model.rht_rows(x[None, :], s)[0], oracle.rht16(x, s))


def test_rht_integer_inputs_are_exact():
    rng = np.random.default_rng(4)
    x = rng.integers(-1000, 1000, 16).astype(np.float32)
    s = 0x3C5A
    ref = 0.25 * H16 @ (_signs_vec(s) * x)
    assert np.array_equal(oracle.rht16(x, s).astype(np.float64), ref)


def test_rht_is_orthogonal_and_invertible():
    rng = np.random.default_rng(5)
    s = oracle.rht_signs(1)
    x = rng.standard_normal(16).astype(np.float32)
    y = oracle.rht16(x, s).astype(np.float64)
    assert abs(np.dot(y, y) - np.dot(x.astype(np.float64), x)) < 1e-5 * np.dot(x, x)
    # (1/4 H D)^-1 = D (1/4 H): transform with no signs, then apply D
    back = _signs_vec(s) * oracle.rht16(y.astype(np.float32), 0).astype(np.float64)
    assert np.max(np.abs(back - x)) < 1e-5


def test_rht_preserves_weight_gradient_dot_products():
    """Both Wgrad operands transformed with the same signs along the token
    dimension: sum_t y_dY[t] y_X[t] equals sum_t dY[t] X[t]."""
    rng = np.random.default_rng(6)
    s = oracle.rht_signs(7)
    for _ in range(50):
        a = rng.standard_normal(16).astype(np.float32)
        b = rng.standard_normal(16).astype(np.float32)
        ya, yb = oracle.rht16(a, s), oracle.rht16(b, s)
        ref = float(np.dot(a.astype(np.float64), b))
        got = float(np.dot(ya.astype(np.float64), yb))
        assert abs(got - ref) < 1e-5 * (np.linalg.norm(a) * np.linalg.norm(b))


def test_rht_spreads_a_single_outlier_evenly():
    """A lone outlier of size M becomes 16 values of magnitude M/4: the
    max/rms ratio drops from 4 to 1."""
    x = np.zeros(16, np.float32)
    x[5] = 1000.0
    y = oracle.rht16(x, oracle.rht_signs(3))
    assert np.all(np.abs(y) == 250.0)
