"""The allocation-free BF16 GEMM (nvfp4_gemm_bf16_noalloc: the K-split
workspace is the library's own per-GPU array) against nvfp4_gemm_bf16 with a
caller workspace: outputs and amax bit for bit, on two calls in a row, the
second with a smaller input (the array keeps the first call's partials and
tickets; each call clears its tickets first), then a shape with no split."""
import numpy as np
import pytest
import torch

import bit_microscaled_numerics_amd as nv
from bit_microscaled_numerics_amd import inputs
from parity import say

pytestmark = pytest.mark.gpu


def _ops(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = inputs.normal(g, M, K, 1.0, 0.001, 50.0)
    w = inputs.normal(g, N, K, 0.02)
    return nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda())


def _both(M, N, K, seed):
    qa, qb = _ops(M, N, K, seed)
    ref = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    got = torch.full((M, N), -1.0, dtype=torch.bfloat16, device="cuda")
    am_ref = torch.empty(1, dtype=torch.float32, device="cuda")
    am_got = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    ws = nv.gemm_bf16_workspace(M, N, K, "cuda")
    nv.nvfp4_gemm_bf16(qa, qb, ref, N, am_ref, ws)
    nv.nvfp4_gemm_bf16_noalloc(qa, qb, got, N, am_got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (M, N, K)
    assert torch.equal(am_got, am_ref), (M, N, K)
    return ws is not None


def test_noalloc_matches_workspace_variant_twice():
    say("gemm bf16 noalloc", (22 * 256, 16 * 256, 512))
    assert _both(22 * 256, 16 * 256, 512, 1)        # K-split tail (96 tiles)
    say("gemm bf16 noalloc, smaller", (17 * 256, 16 * 256, 512))
    assert _both(17 * 256, 16 * 256, 512, 2)        # smaller: N x K split tail (16 tiles)
    say("gemm bf16 noalloc, no split", (272, 144, 512))
    assert not _both(272, 144, 512, 3)


def test_noalloc_rejects_nothing_on_this_device():
    """Every shape's workspace fits the library's array on a 256-CU device;
    the array's size is what the header states."""
    assert nv.load_library().nvfp4_gemm_bf16_noalloc_max_bytes() == 128 * 2 * 65536 * 4 + 512
    for M, N, K in [(8192, 5120, 20480), (8192, 20480, 5120), (5120, 20480, 8192),
                    (22 * 256, 16 * 256, 512), (33 * 256, 4 * 256, 1024)]:
        n = nv.nvfp4_gemm_bf16_workspace_bytes(M, N, K)
        assert 0 <= n <= nv.load_library().nvfp4_gemm_bf16_noalloc_max_bytes(), (M, N, K, n)
