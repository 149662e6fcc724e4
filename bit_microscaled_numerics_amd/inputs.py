"""Seeded synthetic inputs for the NVFP4 linear-layer workloads.

This module only draws random tensors; it contains none of the quantization
or GEMM arithmetic.  Tests and the benchmark hand the same host bytes to the
GPU library and to the CPU oracle.

Shapes follow the 12B hybrid Mamba-Transformer linear layers of "Pretraining
Large Language Models with NVFP4" (summary page, model paragraph: sequence
length 8192) at hidden 5120 / FFN 20480.  Distributions: activations N(0,1)
with a sparse set of large outliers, weights N(0, 0.02), gradients
N(0, 1e-3) or heavy-tailed (Student-t, 3 degrees of freedom, scaled).

Recipe (all draws on the CPU with ``torch.Generator().manual_seed(seed)``,
in the order listed; values are formed in float32 and rounded once to bf16):
  * normal(std):        std * N(0,1)
  * outliers(p, k):     a Bernoulli(p) mask from the same generator, masked
                        entries multiplied by k before the bf16 cast
  * student_t3(scale):  scale * z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), the
                        textbook construction of a t variate with 3 dof from
                        four standard normals
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal(g: torch.Generator, rows: int, cols: int, std: float = 1.0,
           outlier_p: float = 0.0, outlier_k: float = 1.0) -> torch.Tensor:
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if outlier_p > 0.0:
        mask = torch.rand(rows, cols, generator=g, dtype=torch.float32) < outlier_p
        x = torch.where(mask, x * outlier_k, x)
    return x.to(torch.bfloat16)


def student_t3(g: torch.Generator, rows: int, cols: int, scale: float = 1.0) -> torch.Tensor:
    z0 = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    chi = torch.zeros(rows, cols, dtype=torch.float32)
    for _ in range(3):
        z = torch.randn(rows, cols, generator=g, dtype=torch.float32)
        chi.addcmul_(z, z)
    t = z0 / torch.sqrt(chi / 3.0)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(torch.bfloat16)


@dataclass
class Workload:
    """Named tensors (bf16, CPU, row-major) plus the quantization recipe."""
    name: str
    tensors: dict = field(default_factory=dict)
    notes: str = ""


def single_fprop(seed: int = 0) -> Workload:
    """Single Fprop at 256x512x512: X 1D RTN (0.1% outliers x50), W 2D RTN."""
    g = _gen(seed)
    x = normal(g, 256, 512, 1.0, 0.001, 50.0)
    w = normal(g, 512, 512, 0.02)
    return Workload("single_fprop_256x512x512", {"X": x, "W": w},
                    "Y = Q(X) Q(W)^T, X rowwise RTN, W 2D RTN")


def wgrad_rht_sr(seed: int = 0) -> Workload:
    """Wgrad with RHT + SR: dY 4096x1024 = 1e-3 * t3, X 4096x1024 N(0,1)."""
    g = _gen(seed)
    dy = student_t3(g, 4096, 1024, 1e-3)
    x = normal(g, 4096, 1024, 1.0)
    return Workload("wgrad_rht_sr_1024x1024x4096", {"dY": dy, "X": x},
                    "dW = Q(RHT(dY))^T Q(RHT(X)), both SR, K = 4096 tokens")


def ffn_up(seed: int = 0, tokens: int = 8192, hidden: int = 5120, ffn: int = 20480) -> Workload:
    """FFN up-projection Fprop + Dgrad: X [tokens][hidden], W [ffn][hidden],
    dY [tokens][ffn]."""
    g = _gen(seed)
    x = normal(g, tokens, hidden, 1.0, 0.001, 100.0)
    w = normal(g, ffn, hidden, 0.02)
    dy = normal(g, tokens, ffn, 1e-3)
    return Workload(f"ffn_up_{tokens}x{hidden}x{ffn}", {"X": x, "W": w, "dY": dy},
                    "Fprop X rowwise RTN x W 2D; Dgrad dY rowwise SR x W^T")


def ffn_down(seed: int = 0, tokens: int = 8192, hidden: int = 5120, ffn: int = 20480) -> Workload:
    """FFN down-projection fwd+bwd triple: X [tokens][ffn], W [hidden][ffn],
    dY [tokens][hidden]."""
    g = _gen(seed)
    x = normal(g, tokens, ffn, 1.0, 0.001, 100.0)
    w = normal(g, hidden, ffn, 0.02)
    dy = normal(g, tokens, hidden, 1e-3)
    return Workload(f"ffn_down_{tokens}x{ffn}x{hidden}", {"X": x, "W": w, "dY": dy},
                    "Fprop/Dgrad/Wgrad, W 2D, X/dY 1D, SR on dY, RHT on Wgrad inputs")


def sweep_tensors(seed: int = 0, rows: int = 32768, cols: int = 8192) -> Workload:
    """Quantize-only sweep: an N(0,1) tensor and a Student-t(3) tensor."""
    g = _gen(seed)
    a = normal(g, rows, cols, 1.0)
    b = student_t3(g, rows, cols, 1.0)
    return Workload(f"sweep_{rows}x{cols}", {"normal": a, "t3": b},
                    "1D/2D x RTN/SR x RHT on/off")


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (a view, no arithmetic)."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
