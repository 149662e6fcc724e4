"""The GEMM over every E4M3 block-scale code, including the subnormal codes
1..7 and the zero code, through the C ABI.

Operands are built on the host directly as codes and scales (the GEMM's
inputs), so the scales can take values no quantizer of the test tensors
would produce.  With one scale code per row, the tolerance bound of entry
(m, n) is T = s_a s_b E_m E_n sum |q_a q_b|: a wrong decode of any scale
(the kernels take E's power of two from the FP4 -> FP16 convert and multiply
by its mantissa) would miss by at least a sixteenth of T, and a zero scale
must give an exact zero.  Rows 0..255 of A take codes m % 127 and rows of B
codes (n + 50) % 127, so every pair of codes meets.  A second form cycles
the codes along K inside every row (block indexing).  Fprop-like 1D
operands take the fast path (K a multiple of 256, K-contiguous dword
scales) and the general kernel (K % 64 != 0, byte scales); the Dgrad operand
is a 2D weight read through its transposed codes, with transposed scales
and with the untransposed scale array under swapped strides ("Pretraining
Large Language Models with NVFP4", format paragraph: E2M1 elements, one E4M3
scale per 16, an FP32 tensor scale; NVIDIA blog, 2D block quantization)."""
import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
from parity import assert_gemm_close, say

pytestmark = pytest.mark.gpu


def _codes(rng, rows, k):
    return rng.integers(0, 256, (rows, k // 2), dtype=np.uint8)


def _row_scales(rows, k, first):
    return np.repeat(((np.arange(rows) + first) % 127).astype(np.uint8)[:, None], k // 16, axis=1)


def _cycling_scales(rows, nb, a, b):
    return ((np.arange(rows)[:, None] * a + np.arange(nb)[None, :] * b) % 127).astype(np.uint8)


def _pair(codes, scales, ss_row, ss_k, blk, ts, rows, k, codes_t=None):
    """(device operand, oracle operand) of the same bytes."""
    dev = nv.NVFP4Tensor(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                         torch.tensor([ts], dtype=torch.float32).cuda(),
                         torch.zeros(1, dtype=torch.float32).cuda(), rows, k, blk, ss_row, ss_k)
    orc = oracle.Operand(codes, scales, ss_row, ss_k, blk, float(np.float32(ts)), rows, k,
                         0.0, codes_t)
    return dev, orc


def _run(a, b, name):
    (ga, oa), (gb, ob) = a, b
    say("gemm scale codes", name, ga.rows, gb.rows, ga.k)
    c = nv.gemm(ga, gb)
    torch.cuda.synchronize()
    ref, t = oracle.gemm(oa, ob)
    got = c.cpu().numpy()
    assert np.all(got[t == 0] == 0), f"{name}: zero-scale entries not exactly zero"
    assert_gemm_close(got, ref, t, name)


@pytest.mark.parametrize("k", [1024, 1008, 1040])
def test_every_scale_code_pair(k):
    """K = 1024: fast path; 1008 (63 blocks: byte scales) and 1040 (K % 64
    = 16): the general kernel."""
    rng = np.random.default_rng(k)
    M = N = 256
    a = _pair(_codes(rng, M, k), _row_scales(M, k, 0), k // 16, 1, 1, 0.37, M, k)
    b = _pair(_codes(rng, N, k), _row_scales(N, k, 50), k // 16, 1, 1, 1.9e-3, N, k)
    _run(a, b, f"row codes K={k}")


@pytest.mark.parametrize("k", [1024, 1008])
def test_scale_codes_cycling_along_k(k):
    rng = np.random.default_rng(k + 1)
    M, N = 272, 288
    a = _pair(_codes(rng, M, k), _cycling_scales(M, k // 16, 7, 13), k // 16, 1, 1, 2.5e3, M, k)
    b = _pair(_codes(rng, N, k), _cycling_scales(N, k // 16, 11, 5), k // 16, 1, 1, 6.1e-5, N, k)
    _run(a, b, f"cycling K={k}")


def _nibble_transpose(codes: np.ndarray) -> np.ndarray:
    """codes [R][C/2] (low nibble = even column) -> [C][R/2]."""
    R = codes.shape[0]
    full = np.empty((R, codes.shape[1] * 2), np.uint8)
    full[:, 0::2], full[:, 1::2] = codes & 0xF, codes >> 4
    t = np.ascontiguousarray(full.T)
    return (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("scales_form", ["scales_t", "swapped strides"])
def test_dgrad_weight_every_scale_code(scales_form):
    """dX = dY W: A = dY [M][R] with one code per row, B = the 2D weight W
    [R][C] read as [C][R] through its transposed codes; W's 16x16 tiles
    cycle through all 127 codes."""
    rng = np.random.default_rng(5)
    M, R, C = 256, 1024, 512
    w_codes = _codes(rng, R, C)
    w_sc = _cycling_scales(R // 16, C // 16, 9, 4)        # [R/16][C/16]
    w_t = _nibble_transpose(w_codes)                       # [C][R/2]
    ts_w = 0.021
    if scales_form == "scales_t":
        sct = np.ascontiguousarray(w_sc.T)                 # [C/16][R/16]
        gb = _pair(w_t, sct, R // 16, 1, 16, ts_w, C, R)[0]
    else:
        gb = _pair(w_t, w_sc, 1, C // 16, 16, ts_w, C, R)[0]
    ob = _pair(w_codes, w_sc, C // 16, 1, 16, ts_w, R, C, codes_t=w_t)[1].transposed()
    a = _pair(_codes(rng, M, R), _row_scales(M, R, 3), R // 16, 1, 1, 0.9, M, R)
    _run(a, (gb, ob), f"dgrad {scales_form}")
