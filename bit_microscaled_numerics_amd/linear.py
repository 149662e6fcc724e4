"""An NVFP4 linear layer for training: Fprop, Dgrad and Wgrad on the library's
quantizers and GEMMs, with the recipe of "Pretraining Large Language Models
with NVFP4" (summary page, recipe paragraph) and "NVFP4 Trains with Precision
of 16-Bit and Speed and Efficiency of 4-Bit" (method section):

  Fprop  Y  = Q1d(X) Q2d(W)^T               X rowwise, RTN; W 16x16 blocks, RTN
  Dgrad  dX = Q1d_SR(dY) Q2d(W)             the same quantized W, read transposed
  Wgrad  dW = Q_RHT,SR(dY)^T Q_RHT(X)       16-point RHT along the tokens on both
                                            Wgrad inputs, SR on the gradient

plus the fake-quantization ("QDQ") reference of the same layer: identical
quantization, then dequantize and multiply in FP32 -- the way a QDQ
simulation of low-precision training runs ("NVFP4：让大模型从零预训练跑在4位浮点上",
sections 4.1 and 5.2), for layer-by-layer comparison.  Everything runs on the
GPU through the C ABI; there is no CPU path (CPU tensors are rejected).

Random streams: one Philox key per call (seed + step); dY's rowwise SR uses
stream 0, the Wgrad operand of dY stream 1; the RHT signs come from rht_seed.

Opt-in variant (``rht_fprop_dgrad=True``): the 16-point RHT along K on Fprop
and Dgrad as well -- the transform may be applied to the linear layers in the
forward and the backward pass (NVIDIA blog, Hadamard-transforms section),
though the recipe keeps it to Wgrad and leaves Fprop / Dgrad with it
unvalidated ("Pretraining Large Language Models with NVFP4", summary page,
limitations paragraph).  A transform along K mixes 16 weights of a row, which
2D 16x16 weight scaling cannot follow, so W is then quantized 1D along the K
of each GEMM:

  Fprop  Y  = Q_RHT(X) Q_RHT(W)^T           both transformed along F (rows)
  Dgrad  dX = Q_RHT,SR(dY) Q_RHT(W^T)^T     both along H (dY's rows, W's columns)
  Wgrad  as above
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (NVFP4_ROWWISE, NVFP4Tensor, dequantize, gemm, quantize_1d, quantize_2d,
               rht_quantize)


@dataclass
class Seeds:
    rht: int = 1
    sr: int = 1


def _check(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise RuntimeError(f"{name} must be a GPU tensor (the NVFP4 path has no CPU fallback)")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")


def fprop(x: torch.Tensor, w: torch.Tensor):
    """Y = Q1d(X) Q2d(W)^T in FP32; returns (y, quantized W for Dgrad)."""
    qw = quantize_2d(w)
    return gemm(quantize_1d(x), qw), qw


def dgrad(dy: torch.Tensor, qw: NVFP4Tensor, sr_seed: int) -> torch.Tensor:
    """dX = Q1d_SR(dY) Q2d(W) in FP32 (W read through its transposed codes)."""
    return gemm(quantize_1d(dy, sr_seed=sr_seed, stream_id=0), qw.t())


def fprop_rht(x: torch.Tensor, w: torch.Tensor, rht_seed: int) -> torch.Tensor:
    """Y = Q_RHT(X) Q_RHT(W)^T in FP32, both transformed along F (their rows)."""
    return gemm(rht_quantize(x, rht_seed, axis=NVFP4_ROWWISE),
                rht_quantize(w, rht_seed, axis=NVFP4_ROWWISE))


def dgrad_rht(dy: torch.Tensor, w: torch.Tensor, rht_seed: int, sr_seed: int) -> torch.Tensor:
    """dX = Q_RHT,SR(dY) Q_RHT(W^T)^T in FP32, both transformed along H: dY
    along its rows, W through its quantized transpose."""
    return gemm(rht_quantize(dy, rht_seed, sr_seed=sr_seed, stream_id=0, axis=NVFP4_ROWWISE),
                rht_quantize(w, rht_seed))


def wgrad(dy: torch.Tensor, x: torch.Tensor, rht_seed: int, sr_seed: int) -> torch.Tensor:
    """dW = Q_RHT,SR(dY)^T Q_RHT(X) in FP32 (RHT along the tokens)."""
    return gemm(rht_quantize(dy, rht_seed, sr_seed=sr_seed, stream_id=1), rht_quantize(x, rht_seed))


def linear_fwd_bwd(x, w, dy, rht_seed: int, sr_seed: int, rht_fprop_dgrad: bool = False):
    """(Y, dX, dW) of one NVFP4 linear layer in FP32 (bf16 inputs)."""
    for t, n in ((x, "x"), (w, "w"), (dy, "dy")):
        _check(t, n)
    x, w, dy = x.contiguous(), w.contiguous(), dy.contiguous()
    if rht_fprop_dgrad:
        return (fprop_rht(x, w, rht_seed), dgrad_rht(dy, w, rht_seed, sr_seed),
                wgrad(dy, x, rht_seed, sr_seed))
    y, qw = fprop(x, w)
    return y, dgrad(dy, qw, sr_seed), wgrad(dy, x, rht_seed, sr_seed)


class NVFP4LinearFunction(torch.autograd.Function):
    """y = x w^T with NVFP4 operands; x [T][F] bf16, w [H][F] bf16 -> y [T][H]
    FP32.  Gradients are returned in bf16 (the input dtype)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, rht_seed: int, sr_seed: int,
                rht_fprop_dgrad: bool = False):
        _check(x, "x")
        _check(w, "w")
        x, w = x.contiguous(), w.contiguous()
        if rht_fprop_dgrad:
            y, qw = fprop_rht(x, w, rht_seed), None
            ctx.save_for_backward(x, w)
        else:
            y, qw = fprop(x, w)
            ctx.save_for_backward(x)
        ctx.qw = qw
        ctx.seeds = (rht_seed, sr_seed)
        ctx.rht_fprop_dgrad = rht_fprop_dgrad
        return y

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x = ctx.saved_tensors[0]
        rht_seed, sr_seed = ctx.seeds
        dy = dy.to(torch.bfloat16).contiguous()
        if ctx.rht_fprop_dgrad:
            dx = dgrad_rht(dy, ctx.saved_tensors[1], rht_seed, sr_seed)
        else:
            dx = dgrad(dy, ctx.qw, sr_seed)
        dw = wgrad(dy, x, rht_seed, sr_seed)
        return dx.to(torch.bfloat16), dw.to(torch.bfloat16), None, None, None


class NVFP4Linear(torch.nn.Module):
    """A bias-free linear layer whose three GEMMs run in NVFP4.  Each forward
    call draws a fresh SR key (seeds.sr + call index)."""

    def __init__(self, in_features: int, out_features: int, seeds: Seeds | None = None,
                 device=None, rht_fprop_dgrad: bool = False):
        super().__init__()
        self.weight = torch.nn.Parameter(
            torch.empty(out_features, in_features, dtype=torch.bfloat16, device=device))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.seeds = seeds or Seeds()
        self.rht_fprop_dgrad = rht_fprop_dgrad
        self.calls = 0

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        sr = self.seeds.sr + self.calls
        self.calls += 1
        return NVFP4LinearFunction.apply(x, self.weight, self.seeds.rht, sr, self.rht_fprop_dgrad)


@dataclass
class QDQResult:
    y: torch.Tensor
    dx: torch.Tensor
    dw: torch.Tensor


def qdq_reference(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, rht_seed: int,
                  sr_seed: int, rht_fprop_dgrad: bool = False) -> QDQResult:
    """The same layer by fake quantization: the operands quantized exactly as
    NVFP4LinearFunction does (same seeds and streams), dequantized to FP32, and
    multiplied with FP32 matmul.  The RHT operands are dequantized in the
    transformed domain; (H D / 4)^T (H D / 4) = I makes their product dY^T X
    (and X W^T, dY W when the transform is on Fprop / Dgrad too)."""
    _check(x, "x")
    _check(w, "w")
    _check(dy, "dy")
    x, w, dy = x.contiguous(), w.contiguous(), dy.contiguous()
    if rht_fprop_dgrad:
        qx = rht_quantize(x, rht_seed, axis=NVFP4_ROWWISE)
        qwr = rht_quantize(w, rht_seed, axis=NVFP4_ROWWISE)
        y = dequantize(qx) @ dequantize(qwr).t().contiguous()
        qdy = rht_quantize(dy, rht_seed, sr_seed=sr_seed, stream_id=0, axis=NVFP4_ROWWISE)
        dx = dequantize(qdy) @ dequantize(rht_quantize(w, rht_seed)).t().contiguous()
    else:
        qx, qw = quantize_1d(x), quantize_2d(w)
        y = dequantize(qx) @ dequantize(qw).t().contiguous()
        qdy = quantize_1d(dy, sr_seed=sr_seed, stream_id=0)
        dx = dequantize(qdy) @ dequantize(qw)
    qdy_t = rht_quantize(dy, rht_seed, sr_seed=sr_seed, stream_id=1)
    qx_t = rht_quantize(x, rht_seed)
    dw = dequantize(qdy_t) @ dequantize(qx_t).t().contiguous()
    return QDQResult(y, dx, dw)
