"""The NVFP4 training linear layer (Fprop / Dgrad / Wgrad with the recipe's
quantizations) and its fake-quantization reference, on the GPU: the FP32
outputs against the oracle's exact products of the same quantized operands,
the autograd module against the functional form, the QDQ reference against
the oracle, and the layer's agreement with the unquantized product (cosine
similarity, the quality measure of "NVFP4：让大模型从零预训练跑在4位浮点上",
section 4.2)."""
import numpy as np
import pytest
import torch

import oracle
from bit_microscaled_numerics_amd import inputs
from bit_microscaled_numerics_amd import linear as L
from parity import assert_gemm_close, say

pytestmark = pytest.mark.gpu
RHT, SR = 3, 11


def _layer_inputs(T, F, H, seed=0):
    g = torch.Generator().manual_seed(seed)
    x = inputs.normal(g, T, F, 1.0, 0.001, 50.0)
    w = inputs.normal(g, H, F, 0.02)
    dy = inputs.student_t3(g, T, H, 1e-3)
    return x, w, dy


def _oracle_products(x, w, dy):
    ox = oracle.quantize(x, oracle.ROWWISE)
    ow = oracle.quantize(w, oracle.TWO_D, with_codes_t=True)
    ody = oracle.quantize(dy, oracle.ROWWISE, sr_seed=SR, stream_id=0)
    ody_t = oracle.quantize(dy, oracle.COLWISE, rht_seed=RHT, sr_seed=SR, stream_id=1)
    ox_t = oracle.quantize(x, oracle.COLWISE, rht_seed=RHT)
    return oracle.gemm(ox, ow), oracle.gemm(ody, ow.transposed()), oracle.gemm(ody_t, ox_t)


@pytest.mark.parametrize("tfh", [(256, 384, 192), (528, 272, 144)])
def test_functional_matches_oracle(tfh):
    T, F, H = tfh
    x, w, dy = _layer_inputs(T, F, H)
    say("linear fwd/bwd", tfh)
    y, dx, dw = L.linear_fwd_bwd(x.cuda(), w.cuda(), dy.cuda(), RHT, SR)
    torch.cuda.synchronize()
    (cy, ty), (cdx, tdx), (cdw, tdw) = _oracle_products(x, w, dy)
    assert_gemm_close(y.cpu().numpy(), cy, ty, "Y")
    assert_gemm_close(dx.cpu().numpy(), cdx, tdx, "dX")
    assert_gemm_close(dw.cpu().numpy(), cdw, tdw, "dW")


def test_autograd_module_matches_functional():
    T, F, H = 256, 384, 192
    x, w, dy = _layer_inputs(T, F, H, seed=1)
    layer = L.NVFP4Linear(F, H, L.Seeds(rht=RHT, sr=SR), device="cuda")
    with torch.no_grad():
        layer.weight.copy_(w.cuda())
    xd = x.cuda().requires_grad_(True)
    y = layer(xd)
    y.backward(dy.cuda().float())
    torch.cuda.synchronize()
    y2, dx2, dw2 = L.linear_fwd_bwd(x.cuda(), w.cuda(), dy.cuda(), RHT, SR)
    assert torch.equal(y, y2)
    assert torch.equal(xd.grad, dx2.to(torch.bfloat16))
    assert torch.equal(layer.weight.grad, dw2.to(torch.bfloat16))
    assert layer.calls == 1


def test_qdq_reference_matches_oracle():
    T, F, H = 256, 384, 192
    x, w, dy = _layer_inputs(T, F, H, seed=2)
    torch.backends.cuda.matmul.allow_tf32 = False
    r = L.qdq_reference(x.cuda(), w.cuda(), dy.cuda(), RHT, SR)
    torch.cuda.synchronize()
    (cy, ty), (cdx, tdx), (cdw, tdw) = _oracle_products(x, w, dy)
    # FP32 matmul of exactly representable values: the same bound as the GEMMs
    assert_gemm_close(r.y.cpu().numpy(), cy, ty, "QDQ Y")
    assert_gemm_close(r.dx.cpu().numpy(), cdx, tdx, "QDQ dX")
    assert_gemm_close(r.dw.cpu().numpy(), cdw, tdw, "QDQ dW")


def test_layer_tracks_unquantized_product():
    """Cosine similarity of the NVFP4 layer's Y, dX, dW with the unquantized
    FP32 products on heavy-tailed gradients (the RHT + SR Wgrad included).
    A sanity bound, not a parity bar: a wrong operand, transpose or seed gives
    a cosine near 0; the measured values (~0.985-0.995) are reported by the
    benchmark's quality section."""
    T, F, H = 1024, 1024, 512
    x, w, dy = _layer_inputs(T, F, H, seed=3)
    y, dx, dw = L.linear_fwd_bwd(x.cuda(), w.cuda(), dy.cuda(), RHT, SR)
    xf, wf, dyf = x.float().cuda(), w.float().cuda(), dy.float().cuda()
    ref = {"Y": xf @ wf.t().contiguous(), "dX": dyf @ wf, "dW": dyf.t().contiguous() @ xf}
    got = {"Y": y, "dX": dx, "dW": dw}
    for k in ref:
        cos = torch.nn.functional.cosine_similarity(got[k].flatten(), ref[k].flatten(), dim=0)
        say("cosine", k, float(cos))
        assert float(cos) > 0.97, (k, float(cos))


def _oracle_products_rht(x, w, dy):
    """Fprop and Dgrad with the transform along K on both operands (W 1D)."""
    ox = oracle.quantize(x, oracle.ROWWISE, rht_seed=RHT)
    ow = oracle.quantize(w, oracle.ROWWISE, rht_seed=RHT)
    ody = oracle.quantize(dy, oracle.ROWWISE, rht_seed=RHT, sr_seed=SR, stream_id=0)
    owt = oracle.quantize(w, oracle.COLWISE, rht_seed=RHT)
    return oracle.gemm(ox, ow), oracle.gemm(ody, owt)


@pytest.mark.parametrize("tfh", [(256, 384, 192), (528, 272, 144)])
def test_rht_fprop_dgrad_matches_oracle(tfh):
    """The opt-in layer with the 16-point RHT along K on Fprop and Dgrad too
    (NVIDIA blog, Hadamard transforms; left unvalidated by the recipe,
    "Pretraining Large Language Models with NVFP4", limitations paragraph):
    functional form, autograd module and QDQ reference against the oracle."""
    T, F, H = tfh
    x, w, dy = _layer_inputs(T, F, H, seed=4)
    say("linear rht fprop/dgrad", tfh)
    y, dx, dw = L.linear_fwd_bwd(x.cuda(), w.cuda(), dy.cuda(), RHT, SR, rht_fprop_dgrad=True)
    torch.backends.cuda.matmul.allow_tf32 = False
    r = L.qdq_reference(x.cuda(), w.cuda(), dy.cuda(), RHT, SR, rht_fprop_dgrad=True)
    layer = L.NVFP4Linear(F, H, L.Seeds(rht=RHT, sr=SR), device="cuda", rht_fprop_dgrad=True)
    with torch.no_grad():
        layer.weight.copy_(w.cuda())
    xd = x.cuda().requires_grad_(True)
    layer(xd).backward(dy.cuda().float())
    torch.cuda.synchronize()
    (cy, ty), (cdx, tdx) = _oracle_products_rht(x, w, dy)
    (_, _), (_, _), (cdw, tdw) = _oracle_products(x, w, dy)
    assert_gemm_close(y.cpu().numpy(), cy, ty, "Y (RHT)")
    assert_gemm_close(dx.cpu().numpy(), cdx, tdx, "dX (RHT)")
    assert_gemm_close(dw.cpu().numpy(), cdw, tdw, "dW")
    assert_gemm_close(r.y.cpu().numpy(), cy, ty, "QDQ Y (RHT)")
    assert_gemm_close(r.dx.cpu().numpy(), cdx, tdx, "QDQ dX (RHT)")
    assert torch.equal(xd.grad, dx.to(torch.bfloat16))
    assert torch.equal(layer.weight.grad, dw.to(torch.bfloat16))
