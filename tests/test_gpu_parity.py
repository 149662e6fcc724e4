"""HIP path vs CPU oracle on the same seeded inputs, through the C ABI.

Quantization (amax, tensor scale, E4M3 scales, codes, transposed codes) must
be bit-exact; the GEMM must be within 1e-5 * sum_k |a_dec * b_dec| of the
exact product for every entry.  Sizes span several workgroup tiles with
ragged tails; the degenerate cases (all-zero tensors, negative zeros, blocks
whose scale underflows, saturating blocks, K = 16) are included."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
from bit_microscaled_numerics_amd import inputs
from parity import assert_gemm_close, assert_gemm_every_entry, assert_operand_equal, say

pytestmark = pytest.mark.gpu

SHAPES = [(16, 16), (48, 80), (256, 512), (272, 144), (528, 400)]


def _tensor(kind: str, rows: int, cols: int, seed: int = 0) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        return inputs.normal(g, rows, cols)
    if kind == "outliers":
        return inputs.normal(g, rows, cols, 1.0, 0.001, 50.0)
    if kind == "t3":
        return inputs.student_t3(g, rows, cols, 1e-3)
    if kind == "zeros":
        return torch.zeros(rows, cols, dtype=torch.bfloat16)
    if kind == "negzeros":
        return -torch.zeros(rows, cols, dtype=torch.bfloat16)
    if kind == "mixed":
        # all-zero blocks, blocks far below the tensor amax (their scale
        # underflows to zero), one large outlier, exact E2M1 midpoints
        x = inputs.normal(g, rows, cols, 1.0).float()
        x[:, :16] = 0.0
        x[0, -1] = 3.0e4
        if cols >= 64:
            x[1::3, 32:48] *= 1e-6
            ties = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0] * 2)
            x[2::5, 48:64] = ties
        return x.to(torch.bfloat16)
    raise ValueError(kind)


KINDS = ["normal", "outliers", "t3", "zeros", "negzeros", "mixed"]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", ["normal", "t3", "mixed"])
def test_amax(shape, kind):
    x = _tensor(kind, *shape)
    say("amax", shape, kind)
    got = nv.amax(x.cuda())
    torch.cuda.synchronize()
    assert float(got.cpu()[0]) == oracle.amax(x)
    say("amax_rht", shape, kind)
    got = nv.amax_rht(x.cuda(), 1234)
    torch.cuda.synchronize()
    assert float(got.cpu()[0]) == oracle.amax_rht(x, 1234)
    say("amax_both", shape, kind)
    plain, rht = nv.amax_both(x.cuda(), 1234)
    torch.cuda.synchronize()
    assert float(plain.cpu()[0]) == oracle.amax(x)
    assert float(rht.cpu()[0]) == oracle.amax_rht(x, 1234)


@pytest.mark.parametrize("where", ["first", "mid", "last"])
def test_amax_several_trips(where):
    """A tensor past the amax kernels' grid cap, so that workgroups take
    several pieces and the last piece is partial.  On 256 CUs 8208x2064 is
    1035 chunks of 16384 elements for the plain and rowwise-RHT scans (three
    per workgroup, the last one 256 elements long) and 132354 micro-tiles for
    the colwise RHT scan (two per thread).  The largest magnitude is planted
    at the start, in chunk 345 (the first workgroup's second chunk there), or
    at the last element."""
    rows, cols = 8208, 2064
    x = inputs.normal(torch.Generator().manual_seed(11), rows, cols).float()
    x[{"first": (0, 0), "mid": (2739, 100), "last": (rows - 1, cols - 1)}[where]] = -900.0
    x = x.to(torch.bfloat16)
    xd = x.cuda()
    say("amax several trips", where)
    plain = nv.amax(xd)
    both = nv.amax_both(xd, 77)
    row = nv.amax_rht(xd, 77, nv.NVFP4_ROWWISE)
    torch.cuda.synchronize()
    assert float(plain.cpu()[0]) == oracle.amax(x) == 900.0
    assert float(both[0].cpu()[0]) == 900.0
    assert float(both[1].cpu()[0]) == oracle.amax_rht(x, 77)
    assert float(row.cpu()[0]) == oracle.amax_rht(x.t().contiguous(), 77)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("axis", [nv.NVFP4_ROWWISE, nv.NVFP4_COLWISE])
@pytest.mark.parametrize("sr", [False, True])
def test_quantize_1d(shape, kind, axis, sr):
    x = _tensor(kind, *shape, seed=1)
    kw = {"sr_seed": 0xC0FFEE_0000_0001, "stream_id": 3} if sr else {}
    say("quantize_1d", shape, kind, axis, sr)
    g = nv.quantize_1d(x.cuda(), axis, **kw)
    torch.cuda.synchronize()
    o = oracle.quantize(x, oracle.COLWISE if axis else oracle.ROWWISE, **kw)
    assert_operand_equal(g, o, f"1d {shape} {kind} axis={axis} sr={sr}")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("sr", [False, True])
def test_rht_quantize(shape, kind, sr):
    x = _tensor(kind, *shape, seed=2)
    kw = {"sr_seed": 77, "stream_id": 1} if sr else {}
    say("rht_quantize", shape, kind, sr)
    g = nv.rht_quantize(x.cuda(), 99, **kw)
    torch.cuda.synchronize()
    o = oracle.quantize(x, oracle.COLWISE, rht_seed=99, **kw)
    assert_operand_equal(g, o, f"rht {shape} {kind} sr={sr}")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("sr", [False, True])
def test_rht_quantize_rowwise(shape, kind, sr):
    """The transform along each row (the Fprop / Dgrad operands' K): amax
    computed and given, RTN and SR."""
    x = _tensor(kind, *shape, seed=3)
    kw = {"sr_seed": 0xABCD_0000_0077, "stream_id": 4} if sr else {}
    say("rht_quantize rowwise", shape, kind, sr)
    xd = x.cuda()
    g = nv.rht_quantize(xd, 99, axis=nv.NVFP4_ROWWISE, **kw)
    am = nv.amax_rht(xd, 99, nv.NVFP4_ROWWISE)
    g2 = nv.rht_quantize(xd, 99, axis=nv.NVFP4_ROWWISE, amax=am, **kw)
    torch.cuda.synchronize()
    o = oracle.quantize(x, oracle.ROWWISE, rht_seed=99, **kw)
    assert_operand_equal(g, o, f"rht rowwise {shape} {kind} sr={sr}")
    assert_operand_equal(g2, o, f"rht rowwise, amax given {shape} {kind} sr={sr}")
    assert float(am.cpu()[0]) == oracle.amax_rht(x.t().contiguous(), 99)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("sr", [False, True])
def test_quantize_row_rht_one_read(shape, kind, sr):
    """Rowwise operand and RHT transpose from one read: each bit-exact with the
    oracle and byte-identical to the two single calls (same seeds, streams)."""
    x = _tensor(kind, *shape, seed=5)
    sr_seed = 31 if sr else None
    say("quantize_row_rht", shape, kind, sr)
    gr, gt = nv.quantize_row_rht(x.cuda(), 99, sr_seed=sr_seed, stream_ids=(0, 1))
    kw0 = {"sr_seed": 31, "stream_id": 0} if sr else {}
    kw1 = {"sr_seed": 31, "stream_id": 1} if sr else {}
    sr_ = nv.quantize_1d(x.cuda(), nv.NVFP4_ROWWISE, **kw0)
    st_ = nv.rht_quantize(x.cuda(), 99, **kw1)
    torch.cuda.synchronize()
    assert_operand_equal(gr, oracle.quantize(x, oracle.ROWWISE, **kw0), f"row {shape} {kind} {sr}")
    assert_operand_equal(gt, oracle.quantize(x, oracle.COLWISE, rht_seed=99, **kw1),
                         f"rht {shape} {kind} {sr}")
    for a, b in ((gr, sr_), (gt, st_)):
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
        assert torch.equal(a.tensor_scale, b.tensor_scale)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("sr", [False, True])
def test_quantize_2d(shape, kind, sr):
    x = _tensor(kind, *shape, seed=3)
    kw = {"sr_seed": 5, "stream_id": 2} if sr else {}
    say("quantize_2d", shape, kind, sr)
    g = nv.quantize_2d(x.cuda(), **kw)
    torch.cuda.synchronize()
    o = oracle.quantize(x, oracle.TWO_D, with_codes_t=True, **kw)
    assert_operand_equal(g, o, f"2d {shape} {kind} sr={sr}")


def test_amax_given_skips_the_scan():
    x = _tensor("normal", 272, 144)
    xd = x.cuda()
    say("amax_given")
    a = nv.amax(xd)
    g1 = nv.quantize_1d(xd, amax=a)
    g2 = nv.quantize_2d(xd, amax=a)
    g3 = nv.rht_quantize(xd, 5, amax=nv.amax_rht(xd, 5))
    torch.cuda.synchronize()
    assert_operand_equal(g1, oracle.quantize(x, oracle.ROWWISE))
    assert_operand_equal(g2, oracle.quantize(x, oracle.TWO_D, with_codes_t=True))
    assert_operand_equal(g3, oracle.quantize(x, oracle.COLWISE, rht_seed=5))
    # a given amax that is not the tensor's own is used as is
    g4 = nv.quantize_1d(xd, amax=float(a.cpu()[0]) * 4)
    torch.cuda.synchronize()
    assert_operand_equal(g4, oracle.quantize(x, oracle.ROWWISE,
                                             amax_given=float(a.cpu()[0]) * 4))


@pytest.mark.parametrize("factor", [1e-3, 1e-30])
def test_given_amax_below_the_data_saturates(factor):
    """A given amax far below the data: block scales saturate at 448 and
    |v| is huge, so every code saturates at +-6 (RTN and SR, 1D and 2D)."""
    x = _tensor("outliers", 272, 144)
    xd = x.cuda()
    a = oracle.amax(x) * factor
    say("amax_given saturation", factor)
    for gq, oq in [
        (nv.quantize_1d(xd, amax=a), oracle.quantize(x, oracle.ROWWISE, amax_given=a)),
        (nv.quantize_1d(xd, sr_seed=3, amax=a),
         oracle.quantize(x, oracle.ROWWISE, sr_seed=3, amax_given=a)),
        (nv.quantize_2d(xd, amax=a),
         oracle.quantize(x, oracle.TWO_D, amax_given=a, with_codes_t=True)),
        (nv.rht_quantize(xd, 2, amax=a),
         oracle.quantize(x, oracle.COLWISE, rht_seed=2, amax_given=a)),
    ]:
        torch.cuda.synchronize()
        assert_operand_equal(gq, oq, f"saturation {factor}")


def test_sr_is_deterministic_and_seeded():
    x = _tensor("normal", 256, 512)
    xd = x.cuda()
    say("sr determinism")
    a = nv.quantize_1d(xd, sr_seed=1)
    b = nv.quantize_1d(xd, sr_seed=1)
    c = nv.quantize_1d(xd, sr_seed=2)
    d = nv.quantize_1d(xd, sr_seed=1, stream_id=1)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes)
    assert not torch.equal(a.codes, c.codes) and not torch.equal(a.codes, d.codes)


@pytest.mark.parametrize("kind", ["normal", "mixed", "zeros"])
def test_dequantize(kind):
    x = _tensor(kind, 272, 144, seed=4)
    say("dequantize", kind)
    for gq, oq in [(nv.quantize_1d(x.cuda()), oracle.quantize(x, oracle.ROWWISE)),
                   (nv.quantize_2d(x.cuda()), oracle.quantize(x, oracle.TWO_D, with_codes_t=True))]:
        got = nv.dequantize(gq).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), oracle.dequantize(oq).view(np.uint32))
    g2 = nv.quantize_2d(x.cuda())
    o2 = oracle.quantize(x, oracle.TWO_D, with_codes_t=True)
    got = nv.dequantize(g2.t()).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.dequantize(o2.transposed()).view(np.uint32))


# ----------------------------------------------------------------------- GEMM
GEMM_SHAPES = [(16, 16, 16), (48, 80, 48), (64, 32, 80), (256, 512, 512), (272, 528, 144),
               (300 // 16 * 16, 400, 1040)]


@pytest.mark.parametrize("mnk", GEMM_SHAPES)
def test_gemm_fprop(mnk):
    M, N, K = mnk
    g = torch.Generator().manual_seed(M + N + K)
    x = inputs.normal(g, M, K, 1.0, 0.001, 50.0)
    w = inputs.normal(g, N, K, 0.02)
    say("gemm fprop", mnk)
    qx, qw = nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda())
    y = nv.gemm(qx, qw)
    torch.cuda.synchronize()
    ox, ow = oracle.quantize(x, oracle.ROWWISE), oracle.quantize(w, oracle.TWO_D, with_codes_t=True)
    c, t = oracle.gemm(ox, ow)
    assert_gemm_close(y.cpu().numpy(), c, t, f"fprop {mnk}")


@pytest.mark.parametrize("mnk", [(48, 80, 64), (256, 512, 512), (272, 144, 528)])
def test_gemm_dgrad_uses_transposed_weight(mnk):
    M, N, K = mnk          # dX [M][N] = dY [M][K] . W [K][N]
    g = torch.Generator().manual_seed(7)
    dy = inputs.normal(g, M, K, 1e-3)
    w = inputs.normal(g, K, N, 0.02)
    say("gemm dgrad", mnk)
    qdy = nv.quantize_1d(dy.cuda(), sr_seed=1)
    qw = nv.quantize_2d(w.cuda())
    dx = nv.gemm(qdy, qw.t())          # codes_t with the transposed scales
    strided = dataclasses.replace(qw, scales_t=None).t()   # codes_t, scales read strided
    assert strided.ss_k != 1
    dx2 = nv.gemm(qdy, strided)
    torch.cuda.synchronize()
    ody = oracle.quantize(dy, oracle.ROWWISE, sr_seed=1)
    ow = oracle.quantize(w, oracle.TWO_D, with_codes_t=True)
    c, t = oracle.gemm(ody, ow.transposed())
    assert_gemm_close(dx.cpu().numpy(), c, t, f"dgrad {mnk}")
    assert_gemm_close(dx2.cpu().numpy(), c, t, f"dgrad strided scales {mnk}")


@pytest.mark.parametrize("tmn", [(64, 48, 80), (4096, 1024, 1024)])
def test_gemm_wgrad_rht_sr(tmn):
    T, F, H = tmn          # dW [F][H] = dY^T [F][T] . X [T][H]
    g = torch.Generator().manual_seed(8)
    dy = inputs.student_t3(g, T, F, 1e-3)
    x = inputs.normal(g, T, H)
    say("gemm wgrad", tmn)
    qdy = nv.rht_quantize(dy.cuda(), 1, sr_seed=1, stream_id=0)
    qx = nv.rht_quantize(x.cuda(), 1, sr_seed=1, stream_id=1)
    dw = nv.gemm(qdy, qx)
    torch.cuda.synchronize()
    ody = oracle.quantize(dy, oracle.COLWISE, rht_seed=1, sr_seed=1, stream_id=0)
    ox = oracle.quantize(x, oracle.COLWISE, rht_seed=1, sr_seed=1, stream_id=1)
    assert_operand_equal(qdy, ody, "wgrad dY")
    assert_operand_equal(qx, ox, "wgrad X")
    c, t = oracle.gemm(ody, ox)
    assert_gemm_close(dw.cpu().numpy(), c, t, f"wgrad {tmn}")


# Which kernel runs: with dword scales (K-contiguous, K % 64 == 0) a K that
# is a multiple of 256 takes the fast path (raw operands loaded straight to
# LDS, whole 4-step trips); other multiples of 64 take the general kernel.
@pytest.mark.parametrize("mnk", [(272, 400, 512), (48, 80, 256), (64, 96, 1280),   # fast path
                                 (272, 528, 320), (256, 256, 192), (64, 48, 704)])  # general
def test_gemm_fast_path_and_fallback(mnk):
    M, N, K = mnk
    g = torch.Generator().manual_seed(M + N + K)
    x = inputs.normal(g, M, K, 1.0, 0.001, 50.0)
    w = inputs.normal(g, N, K, 0.02)
    say("gemm fast/general", mnk)
    qx, qw = nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda())
    y = nv.gemm(qx, qw)
    torch.cuda.synchronize()
    ox, ow = oracle.quantize(x, oracle.ROWWISE), oracle.quantize(w, oracle.TWO_D)
    c, t = oracle.gemm(ox, ow)
    assert_gemm_close(y.cpu().numpy(), c, t, f"fast/general {mnk}")


def test_gemm_padded_scale_rows():
    """Scale rows padded to a pitch that is a multiple of 4 but not of 16
    bytes: the fast path needs 16-byte scale rows, so this K = 512 GEMM takes
    the general kernel; both operands padded alike, result as the oracle's."""
    import dataclasses
    M, N, K = 272, 144, 512
    g = torch.Generator().manual_seed(77)
    x = inputs.normal(g, M, K, 1.0, 0.001, 50.0)
    w = inputs.normal(g, N, K, 0.02)
    say("gemm padded scale rows", (M, N, K))
    qx, qw = nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda())

    def pad(q):
        rows = q.scales.numel() // (K // 16)
        p = torch.zeros(rows, K // 16 + 4, dtype=torch.uint8, device="cuda")
        p[:, :K // 16] = q.scales.view(rows, K // 16)
        return dataclasses.replace(q, scales=p, ss_row=K // 16 + 4, scales_t=None)

    y = nv.gemm(pad(qx), pad(qw))
    torch.cuda.synchronize()
    ox, ow = oracle.quantize(x, oracle.ROWWISE), oracle.quantize(w, oracle.TWO_D)
    c, t = oracle.gemm(ox, ow)
    assert_gemm_close(y.cpu().numpy(), c, t, "padded scale rows")


def test_gemm_ldc_and_zero_operand():
    g = torch.Generator().manual_seed(9)
    x = inputs.normal(g, 48, 64)
    w = torch.zeros(32, 64, dtype=torch.bfloat16)
    say("gemm ldc/zeros")
    qx, qw = nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda())
    out = torch.full((48, 40), 7.0, device="cuda")
    nv.nvfp4_gemm(qx, qw, out, 40)
    torch.cuda.synchronize()
    o = out.cpu()
    assert torch.all(o[:, :32] == 0) and torch.all(o[:, 32:] == 7.0)


def test_single_fprop_config():
    """The 256x512x512 single-Fprop workload, seed 0, end to end."""
    wl = inputs.single_fprop(0)
    x, w = wl.tensors["X"], wl.tensors["W"]
    say("single fprop workload")
    qx, qw = nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda())
    y = nv.gemm(qx, qw)
    torch.cuda.synchronize()
    ox, ow = oracle.quantize(x, oracle.ROWWISE), oracle.quantize(w, oracle.TWO_D, with_codes_t=True)
    assert_operand_equal(qx, ox, "X")
    assert_operand_equal(qw, ow, "W")
    c, t = oracle.gemm(ox, ow)
    assert_gemm_close(y.cpu().numpy(), c, t, "single fprop")


@pytest.mark.parametrize("K", [1024, 768, 1040])
def test_gemm_split_last_round_is_exact_and_deterministic(K):
    """M = 17*256, N = 16*256: 272 tiles on a 256-CU device leave a last
    round of 16 tiles (the last tile-row), which the GEMM cuts into shorter
    pieces.  Check those tiles densely against the exact oracle, the rest on
    samples, and two runs bit for bit.  K = 1024 (16 steps): fast path, four
    pieces per tile (half-width x K halves added into a zeroed output);
    K = 768 (12 steps, halves not whole 4-step trips): fast path, two
    half-width pieces; K = 1040 (not a multiple of 64): general kernel, two
    K halves."""
    M, N = 17 * 256, 16 * 256
    g = torch.Generator().manual_seed(40)
    x = inputs.normal(g, M, K, 1.0, 0.001, 50.0)
    w = inputs.normal(g, N, K, 0.02)
    say("gemm split tail", (M, N, K))
    qx, qw = nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda())
    y1 = nv.gemm(qx, qw)
    y2 = nv.gemm(qx, qw)
    torch.cuda.synchronize()
    c1, c2 = y1.cpu().numpy(), y2.cpu().numpy()
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))
    ox, ow = oracle.quantize(x, oracle.ROWWISE), oracle.quantize(w, oracle.TWO_D)
    rng = np.random.default_rng(1)
    rows = np.concatenate([np.arange(16 * 256, M), rng.integers(0, 16 * 256, 64)])
    cols = np.concatenate([np.arange(0, N, 61), [N - 1]])
    ms, ns = np.meshgrid(rows, cols, indexing="ij")
    ref, t = oracle.gemm_entries(ox, ow, ms.ravel(), ns.ravel())
    assert_gemm_close(c1[ms.ravel(), ns.ravel()], ref, t, "split tail")
    assert_gemm_every_entry(c1, ox, ow, "split tail, every entry")
