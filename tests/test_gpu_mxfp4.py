"""MXFP4 (the comparison format) on the GPU vs the CPU oracle, through the C
ABI: the quantizer bit-exact (codes and E8M0 scales), dequantize bit-exact,
and the GEMM on the scaled FP4 matrix cores within 1e-5 * sum_k |a*b| of the
exact product, over shapes that span several 256 x 256 tiles, ragged M and N,
K with a partial last 256-wide stage, scale rows that are not 4-byte aligned,
the split of a half-empty last round of tiles, and the benchmark's Fprop shape
on sampled entries."""
import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
from bit_microscaled_numerics_amd import inputs
from parity import assert_gemm_close, say

pytestmark = pytest.mark.gpu


def _cases():
    g = torch.Generator().manual_seed(21)
    yield "normal", inputs.normal(g, 96, 256)
    yield "outliers", inputs.normal(g, 64, 512, 1.0, 0.001, 100.0)
    yield "t3", inputs.student_t3(g, 48, 320)
    yield "tiny", inputs.normal(g, 16, 96, 1e-38)
    yield "huge", inputs.normal(g, 16, 128, 1e37)
    z = torch.zeros(16, 64, dtype=torch.bfloat16)
    z[3, 5] = -0.0
    z[4] = -z[4]
    yield "zeros", z
    r = torch.randn(32, 64, generator=g) * torch.exp2(torch.randint(-40, 40, (32, 1), generator=g).float())
    yield "row_scales", r.to(torch.bfloat16)


def assert_mx_equal(q: nv.MXFP4Tensor, o: oracle.MXOperand, name: str):
    gs, gc = q.scales.cpu().numpy(), q.codes.cpu().numpy()
    bad = np.argwhere(gs != o.scales)
    assert bad.size == 0, f"{name}: {len(bad)} scale mismatches, first {bad[:4].tolist()}"
    bad = np.argwhere(gc != o.codes)
    assert bad.size == 0, f"{name}: {len(bad)} code-byte mismatches, first {bad[:4].tolist()}"


@pytest.mark.parametrize("sr", [False, True])
def test_quantize_bit_exact(sr):
    for name, x in _cases():
        say("mx quantize", name, "sr" if sr else "rtn", tuple(x.shape))
        q = nv.mx_quantize(x.cuda(), sr_seed=7 if sr else None, stream_id=2)
        torch.cuda.synchronize()
        o = oracle.mx_quantize(x, sr_seed=7 if sr else None, stream_id=2)
        assert_mx_equal(q, o, name)


def test_dequantize_bit_exact():
    for name, x in _cases():
        q = nv.mx_quantize(x.cuda())
        d = nv.mx_dequantize(q).cpu().numpy()
        o = oracle.mx_dequantize(oracle.mx_quantize(x))
        assert np.array_equal(d.view(np.uint32), o.view(np.uint32)), name


def _operands(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    a = (torch.randn(M, K, generator=g) *
         torch.exp2(torch.randint(-6, 7, (M, 1), generator=g).float())).to(torch.bfloat16)
    b = (torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16)
    return a, b


# (300, 260, 768) and (520, 264, 1280) are ragged in M and N with whole
# 256-K stages (3 and 5 of them: odd counts); (272, 144, 544) and
# (520, 264, 1312) end in a partial stage
@pytest.mark.parametrize("mnk", [(32, 32, 32), (64, 96, 64), (256, 256, 256), (300, 260, 96),
                                 (272, 144, 544), (512, 768, 1024), (520, 264, 1312),
                                 (300, 260, 768), (520, 264, 1280)])
def test_gemm_matches_exact_product(mnk):
    M, N, K = mnk
    a, b = _operands(M, N, K, M + N + K)
    say("mx gemm", mnk)
    qa, qb = nv.mx_quantize(a.cuda()), nv.mx_quantize(b.cuda())
    c = nv.mx_gemm(qa, qb)
    torch.cuda.synchronize()
    oa, ob = oracle.mx_quantize(a), oracle.mx_quantize(b)
    ref, t = oracle.mx_gemm(oa, ob)
    assert_gemm_close(c.cpu().numpy(), ref, t, f"mx gemm {mnk}")


def test_gemm_split_last_round_and_determinism():
    """17 x 16 tiles: the last round is split into two K halves that add into
    a zeroed output; the result is bitwise repeatable."""
    M, N, K = 17 * 256, 16 * 256, 1024
    a, b = _operands(M, N, K, 5)
    say("mx gemm split", (M, N, K))
    qa, qb = nv.mx_quantize(a.cuda()), nv.mx_quantize(b.cuda())
    c1 = nv.mx_gemm(qa, qb)
    c2 = nv.mx_gemm(qa, qb)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    oa, ob = oracle.mx_quantize(a), oracle.mx_quantize(b)
    rng = np.random.default_rng(0)
    ms = np.concatenate([rng.integers(0, M, 3000), np.arange(M - 256, M)])
    ns = np.concatenate([rng.integers(0, N, 3000), rng.integers(0, N, 256)])
    ref, t = oracle.mx_gemm_entries(oa, ob, ms, ns)
    assert_gemm_close(c1.cpu().numpy()[ms, ns], ref, t, "mx gemm split")
    ref, t = oracle.mx_gemm_f64(oa, ob)
    assert_gemm_close(c1.cpu().numpy(), ref, t, "mx gemm split, every entry")


def test_gemm_split_odd_stages():
    """17 x 16 tiles at K = 768 (3 stages): the split last round's halves have
    2 and 1 stages."""
    M, N, K = 17 * 256, 16 * 256, 768
    a, b = _operands(M, N, K, 6)
    say("mx gemm split odd", (M, N, K))
    qa, qb = nv.mx_quantize(a.cuda()), nv.mx_quantize(b.cuda())
    c = nv.mx_gemm(qa, qb)
    torch.cuda.synchronize()
    oa, ob = oracle.mx_quantize(a), oracle.mx_quantize(b)
    rng = np.random.default_rng(2)
    ms = np.concatenate([rng.integers(0, M, 3000), np.arange(M - 256, M)])
    ns = np.concatenate([rng.integers(0, N, 3000), rng.integers(0, N, 256)])
    ref, t = oracle.mx_gemm_entries(oa, ob, ms, ns)
    assert_gemm_close(c.cpu().numpy()[ms, ns], ref, t, "mx gemm split odd")
    ref, t = oracle.mx_gemm_f64(oa, ob)
    assert_gemm_close(c.cpu().numpy(), ref, t, "mx gemm split odd, every entry")


def test_gemm_padded_scale_rows():
    """Scale rows padded to a multiple of 4 bytes (K / 32 = 3 blocks, 4 bytes
    per row) with 0xFF (the E8M0 NaN) in the padding: the padding is never
    read as a block scale."""
    M, N, K = 64, 96, 96
    a, b = _operands(M, N, K, 7)
    say("mx gemm padded scale rows", (M, N, K))
    qa, qb = nv.mx_quantize(a.cuda()), nv.mx_quantize(b.cuda())

    def padded(q):
        sc = torch.full((q.rows, 4), 0xFF, dtype=torch.uint8, device="cuda")
        sc[:, :K // 32] = q.scales
        return nv.MXFP4Tensor(q.codes, sc, q.rows, q.k)

    c = torch.empty(M, N, dtype=torch.float32, device="cuda")
    nv.mxfp4_gemm(padded(qa), padded(qb), c, N)
    torch.cuda.synchronize()
    oa, ob = oracle.mx_quantize(a), oracle.mx_quantize(b)
    ref, t = oracle.mx_gemm(oa, ob)
    cc = c.cpu().numpy()
    assert np.all(np.isfinite(cc))
    assert_gemm_close(cc, ref, t, "mx gemm padded scale rows")


def test_gemm_fprop_shape_sampled():
    """The benchmark's Fprop shape, 8192 x 5120 x 20480, from the FFN
    down-projection tensors quantized as MXFP4; sampled entries on the
    oracle's loop and every entry on its float64 matmul form."""
    wl = inputs.ffn_down(0)
    X, W = wl.tensors["X"], wl.tensors["W"]
    say("mx gemm fprop 8192x5120x20480")
    qx, qw = nv.mx_quantize(X.cuda()), nv.mx_quantize(W.cuda())
    y = nv.mx_gemm(qx, qw)
    torch.cuda.synchronize()
    ox, ow = oracle.mx_quantize(X), oracle.mx_quantize(W)
    assert_mx_equal(qx, ox, "X")
    assert_mx_equal(qw, ow, "W")
    rng = np.random.default_rng(1)
    ms = np.concatenate([[0, 8191, 255, 256], rng.integers(0, 8192, 1500)])
    ns = np.concatenate([[0, 5119, 256, 255], rng.integers(0, 5120, 1500)])
    ref, t = oracle.mx_gemm_entries(ox, ow, ms, ns)
    yc = y.cpu().numpy()
    assert np.all(np.isfinite(yc))
    assert_gemm_close(yc[ms, ns], ref, t, "mx fprop")
    say("mx gemm fprop, every entry")
    ref, t = oracle.mx_gemm_f64(ox, ow)
    assert_gemm_close(yc, ref, t, "mx fprop, every entry")
