"""Parity at the full workload sizes, in the launch configuration bench.py
times: every quantized tensor is compared byte for byte with the oracle over
the whole tensor; GEMM outputs are compared with the oracle's exact product on
sampled entries (all tile corners plus random ones), and every entry with its
float64 form (oracle.gemm_f64, whose own error of about K * 2^-53 * T is far
inside the 1e-5 * T tolerance).  Workloads: the 12B hybrid's FFN up-projection
(Fprop + Dgrad), the FFN down-projection triple (Fprop, Dgrad, Wgrad with
RHT + SR), the 4096-token Wgrad with RHT + SR on heavy-tailed gradients
(full product), and the 32768 x 8192 quantize sweep."""
import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
from bit_microscaled_numerics_amd import inputs
from parity import assert_gemm_close, assert_operand_equal, say

pytestmark = pytest.mark.gpu


def sample_entries(M, N, n_random=1536, seed=0):
    rng = np.random.default_rng(seed)
    edges_m = sorted({0, 1, 31, 32, 127, 128, 255, 256, M // 2, M - 257, M - 256, M - 1})
    edges_n = sorted({0, 1, 31, 32, 127, 128, 255, 256, N // 2, N - 257, N - 256, N - 1})
    em, en = np.meshgrid([m for m in edges_m if 0 <= m < M], [n for n in edges_n if 0 <= n < N])
    ms = np.concatenate([em.ravel(), rng.integers(0, M, n_random)])
    ns = np.concatenate([en.ravel(), rng.integers(0, N, n_random)])
    return ms.astype(np.int64), ns.astype(np.int64)


def check_gemm_sampled(c_dev: torch.Tensor, oa, ob, name):
    c = c_dev.cpu().numpy()
    assert np.all(np.isfinite(c)), f"{name}: non-finite outputs"
    ms, ns = sample_entries(*c.shape)
    ref, t = oracle.gemm_entries(oa, ob, ms, ns)
    assert_gemm_close(c[ms, ns], ref, t, name + " (exact path, sampled entries)")
    say(name, "every entry")
    ref, t = oracle.gemm_f64(oa, ob)
    assert_gemm_close(c, ref, t, name + " (float64 form, every entry)")


def test_ffn_up_fprop_dgrad():
    """X 8192x5120 (0.1% outliers x100) rowwise RTN, W 20480x5120 2D RTN,
    dY 8192x20480 rowwise SR; Fprop 8192x20480x5120, Dgrad 8192x5120x20480."""
    wl = inputs.ffn_up(0)
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    say("ffn_up quantize")
    qx = nv.quantize_1d(X.cuda())
    qw = nv.quantize_2d(W.cuda())
    qdy = nv.quantize_1d(dY.cuda(), sr_seed=1)
    torch.cuda.synchronize()
    ox = oracle.quantize(X, oracle.ROWWISE)
    ow = oracle.quantize(W, oracle.TWO_D, with_codes_t=True)
    ody = oracle.quantize(dY, oracle.ROWWISE, sr_seed=1)
    assert_operand_equal(qx, ox, "X")
    assert_operand_equal(qw, ow, "W")
    assert_operand_equal(qdy, ody, "dY")
    say("ffn_up fprop")
    y = nv.gemm(qx, qw)
    torch.cuda.synchronize()
    check_gemm_sampled(y, ox, ow, "fprop 8192x20480x5120")
    del y
    say("ffn_up dgrad")
    dx = nv.gemm(qdy, qw.t())
    torch.cuda.synchronize()
    check_gemm_sampled(dx, ody, ow.transposed(), "dgrad 8192x5120x20480")


def test_ffn_down_triple():
    """The benchmark step: X 8192x20480, W 5120x20480, dY 8192x5120; Fprop,
    Dgrad, Wgrad with RHT on both Wgrad operands, SR on dY."""
    wl = inputs.ffn_down(0)
    X, W, dY = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    xd, wd, dyd = X.cuda(), W.cuda(), dY.cuda()
    say("ffn_down quantize")
    qx = nv.quantize_1d(xd)
    qw = nv.quantize_2d(wd)
    qdy = nv.quantize_1d(dyd, sr_seed=1)
    qdy_t = nv.rht_quantize(dyd, 1, sr_seed=1, stream_id=1)
    qx_t = nv.rht_quantize(xd, 1)
    torch.cuda.synchronize()
    ox = oracle.quantize(X, oracle.ROWWISE)
    ow = oracle.quantize(W, oracle.TWO_D, with_codes_t=True)
    ody = oracle.quantize(dY, oracle.ROWWISE, sr_seed=1)
    ody_t = oracle.quantize(dY, oracle.COLWISE, rht_seed=1, sr_seed=1, stream_id=1)
    ox_t = oracle.quantize(X, oracle.COLWISE, rht_seed=1)
    for g, o, n in [(qx, ox, "X"), (qw, ow, "W"), (qdy, ody, "dY"), (qdy_t, ody_t, "RHT dY^T"),
                    (qx_t, ox_t, "RHT X^T")]:
        assert_operand_equal(g, o, n)
    say("ffn_down gemms")
    y = nv.gemm(qx, qw)
    torch.cuda.synchronize()
    check_gemm_sampled(y, ox, ow, "fprop 8192x5120x20480")
    del y
    dx = nv.gemm(qdy, qw.t())
    torch.cuda.synchronize()
    check_gemm_sampled(dx, ody, ow.transposed(), "dgrad 8192x20480x5120")
    del dx
    dw = nv.gemm(qdy_t, qx_t)
    torch.cuda.synchronize()
    check_gemm_sampled(dw, ody_t, ox_t, "wgrad 5120x20480x8192")


def test_wgrad_rht_sr_full_product():
    """dY 4096x1024 = 1e-3 t3, X 4096x1024 N(0,1): both RHT + SR along the
    4096 tokens; every entry of dW = dY^T X checked."""
    wl = inputs.wgrad_rht_sr(0)
    dY, X = wl.tensors["dY"], wl.tensors["X"]
    say("wgrad 1024x1024x4096")
    qdy = nv.rht_quantize(dY.cuda(), 1, sr_seed=1, stream_id=0)
    qx = nv.rht_quantize(X.cuda(), 1, sr_seed=1, stream_id=1)
    dw = nv.gemm(qdy, qx)
    torch.cuda.synchronize()
    ody = oracle.quantize(dY, oracle.COLWISE, rht_seed=1, sr_seed=1, stream_id=0)
    ox = oracle.quantize(X, oracle.COLWISE, rht_seed=1, sr_seed=1, stream_id=1)
    assert_operand_equal(qdy, ody, "dY")
    assert_operand_equal(qx, ox, "X")
    c, t = oracle.gemm(ody, ox)
    assert_gemm_close(dw.cpu().numpy(), c, t, "wgrad full")


@pytest.mark.parametrize("dist", ["normal", "t3"])
def test_sweep_32768x8192(dist):
    g = torch.Generator().manual_seed(0)
    if dist == "normal":
        x = inputs.normal(g, 32768, 8192)
    else:
        x = inputs.student_t3(g, 32768, 8192)
    xd = x.cuda()
    cases = [
        ("1d RTN", lambda: nv.quantize_1d(xd), lambda: oracle.quantize(x, oracle.ROWWISE)),
        ("1d SR", lambda: nv.quantize_1d(xd, sr_seed=3, stream_id=2),
         lambda: oracle.quantize(x, oracle.ROWWISE, sr_seed=3, stream_id=2)),
        ("2d RTN", lambda: nv.quantize_2d(xd),
         lambda: oracle.quantize(x, oracle.TWO_D, with_codes_t=True)),
        ("col RTN", lambda: nv.quantize_1d(xd, nv.NVFP4_COLWISE),
         lambda: oracle.quantize(x, oracle.COLWISE)),
        ("RHT SR", lambda: nv.rht_quantize(xd, 4, sr_seed=5),
         lambda: oracle.quantize(x, oracle.COLWISE, rht_seed=4, sr_seed=5)),
    ]
    for name, gpu, orc in cases:
        say("sweep", dist, name)
        gq = gpu()
        torch.cuda.synchronize()
        oq = orc()
        assert_operand_equal(gq, oq, f"{dist} {name}")
        if name in ("1d RTN", "2d RTN"):
            # the whole tensor dequantized, bit for bit (2D also through its
            # transposed view)
            say("sweep", dist, name, "dequantize")
            views = [(gq, oq)] + ([(gq.t(), oq.transposed())] if name == "2d RTN" else [])
            for gv, ov in views:
                d = nv.dequantize(gv)
                torch.cuda.synchronize()
                got = d.cpu().numpy()
                del d
                want = oracle.dequantize(ov)
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
                    f"{dist} {name} dequantize: {int(np.sum(got.view(np.uint32) != want.view(np.uint32)))} differ"
        del gq, oq
