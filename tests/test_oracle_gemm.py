"""Pins of the oracle's NVFP4 GEMM: exact rational arithmetic on tiny cases
(Python fractions), a float64 library matmul of the decoded operands, one-hot
operands, the bound T, and the Fprop / Dgrad / Wgrad operand mappings against
products of dequantized tensors.  CPU only."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import model
from bit_microscaled_numerics_amd import inputs

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def e4m3_frac(code: int) -> Fraction:
    e, m = (code >> 3) & 15, code & 7
    if e == 0:
        return Fraction(m, 512)
    return Fraction(8 + m, 8) * (Fraction(2) ** (e - 7))


def decoded_f64(q: oracle.Operand) -> np.ndarray:
    """q.E as float64 via torch's float8 decode (no oracle arithmetic)."""
    codes = model.unpack(q.codes)[:, :q.k]
    vals = np.where(codes & 8, -1.0, 1.0) * np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[codes & 7]
    r = np.arange(q.rows)[:, None] // q.blk_rows
    k = np.arange(q.k)[None, :] // 16
    sc = q.scales.reshape(-1)[r * q.ss_row + k * q.ss_k]
    E = torch.from_numpy(sc.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    return vals * E


def test_k16_single_block_exact_rational():
    g = torch.Generator().manual_seed(30)
    a = oracle.quantize(inputs.normal(g, 16, 16), oracle.ROWWISE)
    b = oracle.quantize(inputs.normal(g, 16, 16, 0.02), oracle.TWO_D)
    c, t = oracle.gemm(a, b)
    ca = model.unpack(a.codes)
    cb = model.unpack(b.codes)
    for m in range(16):
        for n in range(16):
            acc = Fraction(0)
            tacc = Fraction(0)
            for k in range(16):
                va = GRID[ca[m, k] & 7] * (-1 if ca[m, k] & 8 else 1) * e4m3_frac(int(a.scales[m, 0]))
                vb = GRID[cb[n, k] & 7] * (-1 if cb[n, k] & 8 else 1) * e4m3_frac(int(b.scales[0, 0]))
                acc += va * vb
                tacc += abs(va * vb)
            s = Fraction(a.tensor_scale) * Fraction(b.tensor_scale)
            assert c[m, n] == float(acc * s)
            assert t[m, n] == float(tacc * s)


def test_matches_float64_matmul_of_decoded_operands():
    g = torch.Generator().manual_seed(31)
    x = inputs.normal(g, 48, 96, 1.0, 0.01, 50.0)
    w = inputs.normal(g, 64, 96, 0.02)
    a = oracle.quantize(x, oracle.ROWWISE)
    b = oracle.quantize(w, oracle.TWO_D)
    c, t = oracle.gemm(a, b)
    ref = (decoded_f64(a) @ decoded_f64(b).T) * a.tensor_scale * b.tensor_scale
    tref = (np.abs(decoded_f64(a)) @ np.abs(decoded_f64(b)).T) * a.tensor_scale * b.tensor_scale
    assert np.all(np.abs(c - ref) <= 1e-13 * tref)
    assert np.allclose(t, tref, rtol=1e-13, atol=0)
    assert np.all(t >= np.abs(c))


def test_one_hot_operands_return_single_products():
    """A has one nonzero code per row; the product picks one column of B."""
    K = 64
    x = np.zeros((16, K), np.float32)
    for m in range(16):
        x[m, (5 * m) % K] = 6.0          # amax 6 in every block it sits in
    a = oracle.quantize(torch.from_numpy(x).to(torch.bfloat16), oracle.ROWWISE)
    g = torch.Generator().manual_seed(32)
    b = oracle.quantize(inputs.normal(g, 32, K), oracle.ROWWISE)
    c, _ = oracle.gemm(a, b)
    db = decoded_f64(b)
    da = decoded_f64(a)
    for m in range(16):
        k = (5 * m) % K
        assert c[m].tolist() == (da[m, k] * db[:, k] * a.tensor_scale * b.tensor_scale).tolist()


def test_fprop_dgrad_wgrad_operand_mappings():
    g = torch.Generator().manual_seed(33)
    T, H, F = 64, 32, 48                       # tokens, in-features, out-features
    X = inputs.normal(g, T, H)
    W = inputs.normal(g, F, H, 0.02)
    dY = inputs.normal(g, T, F, 1e-3)
    qx = oracle.quantize(X, oracle.ROWWISE)
    qw = oracle.quantize(W, oracle.TWO_D, with_codes_t=True)
    qdy = oracle.quantize(dY, oracle.ROWWISE, sr_seed=1)
    xh, wh, dyh = (oracle.dequantize(q).astype(np.float64) for q in (qx, qw, qdy))

    # Fprop: Y = X W^T
    y, ty = oracle.gemm(qx, qw)
    assert np.all(np.abs(y - xh @ wh.T) <= 1e-6 * ty)
    # Dgrad: dX = dY W, B = W^T read through the transposed 2D codes
    dx, tdx = oracle.gemm(qdy, qw.transposed())
    assert dx.shape == (T, H)
    assert np.all(np.abs(dx - dyh @ wh) <= 1e-6 * tdx)
    # Wgrad: dW = dY^T X, both quantized along tokens (COLWISE), same RHT signs
    qdy_t = oracle.quantize(dY, oracle.COLWISE, rht_seed=7, sr_seed=1, stream_id=0)
    qx_t = oracle.quantize(X, oracle.COLWISE, rht_seed=7, sr_seed=1, stream_id=1)
    dw, tdw = oracle.gemm(qdy_t, qx_t)
    assert dw.shape == (F, H)
    ref = dY.double().numpy().T @ X.double().numpy()
    # the RHT cancels in the product; what remains is 4-bit quantization noise
    rel = np.linalg.norm(dw - ref) / np.linalg.norm(ref)
    assert rel < 0.25


def test_gemm_entries_equal_full_product():
    g = torch.Generator().manual_seed(34)
    a = oracle.quantize(inputs.normal(g, 32, 64), oracle.ROWWISE)
    b = oracle.quantize(inputs.normal(g, 48, 64), oracle.ROWWISE, sr_seed=3)
    c, t = oracle.gemm(a, b)
    ms = np.array([0, 31, 5, 17])
    ns = np.array([47, 0, 5, 33])
    ce, te = oracle.gemm_entries(a, b, ms, ns)
    assert np.array_equal(ce, c[ms, ns]) and np.array_equal(te, t[ms, ns])


# ---------------------------------------------------------------------------
# The float64 form (decode_exact + a float64 library matmul): the fast form of
# the GEMM for whole full-size products.
# ---------------------------------------------------------------------------

def _wide_range(g, rows, cols, seed_scale=1.0):
    """Rows scaled by 2^0 .. 2^-30 so that the block scales run from the top of
    E4M3 down through its subnormal codes (and to zero) within one tensor."""
    x = inputs.normal(g, rows, cols, seed_scale).float()
    x = x * torch.pow(2.0, -(torch.arange(rows) % 31).float())[:, None]
    return x.to(torch.bfloat16)


def test_decode_exact_equals_independent_decode_every_layout():
    g = torch.Generator().manual_seed(35)
    x = _wide_range(g, 64, 128)
    w = _wide_range(g, 96, 128)
    qs = [oracle.quantize(x, oracle.ROWWISE),
          oracle.quantize(x, oracle.ROWWISE, sr_seed=5),
          oracle.quantize(w, oracle.TWO_D, with_codes_t=True),
          oracle.quantize(x, oracle.COLWISE, rht_seed=3),
          oracle.quantize(x, oracle.COLWISE)]
    qs.append(qs[2].transposed())
    codes_seen = set()
    for q in qs:
        d = oracle.decode_exact(q)
        assert d.shape == (q.rows, q.k) and d.dtype == np.float64
        assert np.array_equal(d, decoded_f64(q))       # values (its zeros are +0)
        codes_seen |= set(np.unique(q.scales).tolist())
    # the scales reached the subnormal E4M3 codes and zero as well as normal ones
    assert {0} | set(range(1, 8)) <= codes_seen and max(codes_seen) >= 0x70


def test_gemm_f64_k16_equals_exact_rational():
    """One block along K: every float64 sum is exact, so the float64 form
    equals the rational result exactly."""
    g = torch.Generator().manual_seed(30)
    a = oracle.quantize(inputs.normal(g, 16, 16), oracle.ROWWISE)
    b = oracle.quantize(inputs.normal(g, 16, 16, 0.02), oracle.TWO_D)
    c, t = oracle.gemm_f64(a, b)
    ce, te = oracle.gemm(a, b)          # itself pinned by the fractions test above
    assert np.array_equal(c, ce) and np.array_equal(t, te)


def test_gemm_f64_within_its_bound_of_the_exact_path():
    """Every mapping, a long K and a wide scale range: |C_f64 - C_exact| is
    inside the float64 summation bound K * 2^-52 * T (far inside 1e-5 * T)."""
    g = torch.Generator().manual_seed(36)
    T_, H, F = 256, 64, 96                     # tokens, in-features, out-features
    X = _wide_range(g, T_, H)
    W = inputs.normal(g, F, H, 0.02)
    dY = inputs.normal(g, T_, F, 1e-3)
    qx = oracle.quantize(X, oracle.ROWWISE)
    qw = oracle.quantize(W, oracle.TWO_D, with_codes_t=True)
    qdy = oracle.quantize(dY, oracle.ROWWISE, sr_seed=1)
    qdy_t = oracle.quantize(dY, oracle.COLWISE, rht_seed=7, sr_seed=1, stream_id=0)
    qx_t = oracle.quantize(X, oracle.COLWISE, rht_seed=7)
    long_a = oracle.quantize(inputs.normal(g, 32, 4096), oracle.ROWWISE, sr_seed=2)
    long_b = oracle.quantize(inputs.normal(g, 48, 4096, 0.05), oracle.ROWWISE)
    for a, b in [(qx, qw), (qdy, qw.transposed()), (qdy_t, qx_t), (long_a, long_b)]:
        c, t = oracle.gemm_f64(a, b)
        ce, te = oracle.gemm(a, b)
        bound = a.k * 2.0 ** -52 * te
        assert np.all(np.abs(c - ce) <= bound)
        assert np.all(np.abs(t - te) <= bound)
        assert np.all(t >= np.abs(c) * (1 - 1e-12))
        # and without the bound the product is the same array
        assert np.array_equal(oracle.gemm_f64(a, b, with_bound=False), c)
