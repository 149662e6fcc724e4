"""The fused GEMM epilogue (BF16 output + max |C|): the BF16 output is exactly
the FP32 output rounded to nearest-even -- on every shape when the K-split
workspace is given (the last round's tiles then split along K as in the FP32
path, both halves' partials meeting in the workspace), and where the FP32 path
computes every tile whole without it; the amax is exactly max |C| over the
written BF16 values; quantizing C with that amax given equals quantizing it
with a computed amax byte for byte; at the benchmark's Fprop shape the BF16
output matches the oracle's exact product within the GEMM tolerance plus BF16
rounding."""
import numpy as np
import pytest
import torch

import oracle
import bit_microscaled_numerics_amd as nv
from bit_microscaled_numerics_amd import inputs
from parity import GEMM_TOL, assert_gemm_every_entry, say

pytestmark = pytest.mark.gpu


def rne_bf16_bits(f32: np.ndarray) -> np.ndarray:
    u = f32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _ops(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = inputs.normal(g, M, K, 1.0, 0.001, 50.0)
    w = inputs.normal(g, N, K, 0.02)
    return nv.quantize_1d(x.cuda()), nv.quantize_2d(w.cuda()), x, w


@pytest.mark.parametrize("mnk", [(48, 80, 64), (272, 144, 528), (512, 768, 1024), (16, 16, 16)])
def test_bf16_is_rounded_fp32_and_amax_exact(mnk):
    M, N, K = mnk
    qa, qb, _, _ = _ops(M, N, K, M + N + K)
    say("gemm bf16", mnk)
    c32 = nv.gemm(qa, qb)
    cb, amax = nv.gemm_bf16(qa, qb)
    torch.cuda.synchronize()
    got = cb.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, rne_bf16_bits(c32.cpu().numpy()))
    mag = (got & 0x7FFF).astype(np.uint32) << 16
    assert float(amax.cpu()[0]) == float(mag.max().view(np.float32))


@pytest.mark.parametrize("mnk", [(22 * 256, 16 * 256, 512),     # 352 tiles: 96 cut in K halves
                                 (17 * 256, 16 * 256, 1024)])   # 272 tiles: 16 cut in 4 pieces
def test_bf16_split_tail_is_rounded_fp32(mnk):
    """Tail tiles cut along K (and N): both halves' FP32 partials meet in the
    workspace, so every entry is the FP32 path's sum rounded; twice, bit for
    bit (the workspace is reused as it comes)."""
    M, N, K = mnk
    qa, qb, _, _ = _ops(M, N, K, M + K)
    say("gemm bf16 split tail", mnk)
    ws = nv.gemm_bf16_workspace(M, N, K, "cuda")
    assert ws is not None and ws.numel() == nv.nvfp4_gemm_bf16_workspace_bytes(M, N, K)
    c32 = nv.gemm(qa, qb)
    cb1, amax = nv.gemm_bf16(qa, qb, workspace=ws)
    cb2, _ = nv.gemm_bf16(qa, qb, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(cb1, cb2)
    got = cb1.cpu().view(torch.int16).numpy().view(np.uint16)
    want = rne_bf16_bits(c32.cpu().numpy())
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:4].tolist())
    mag = (got & 0x7FFF).astype(np.uint32) << 16
    assert float(amax.cpu()[0]) == float(mag.max().view(np.float32))


def test_given_amax_feeds_the_next_quantization():
    qa, qb, _, _ = _ops(256, 512, 256, 3)
    cb, amax = nv.gemm_bf16(qa, qb)
    q_given = nv.quantize_1d(cb, amax=amax)
    q_comp = nv.quantize_1d(cb)
    torch.cuda.synchronize()
    assert torch.equal(q_given.amax, q_comp.amax)
    assert torch.equal(q_given.codes, q_comp.codes)
    assert torch.equal(q_given.scales, q_comp.scales)


def test_fprop_shape_against_oracle():
    wl = inputs.ffn_down(0)
    X, W = wl.tensors["X"], wl.tensors["W"]
    say("gemm bf16 fprop 8192x5120x20480")
    qx, qw = nv.quantize_1d(X.cuda()), nv.quantize_2d(W.cuda())
    cb, amax = nv.gemm_bf16(qx, qw)
    c32 = nv.gemm(qx, qw)
    torch.cuda.synchronize()
    # 640 tiles: the last 128 are cut along K; every entry is the FP32 one rounded
    got = cb.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, rne_bf16_bits(c32.cpu().numpy()))
    del c32
    y = cb.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y))
    assert float(amax.cpu()[0]) == float(np.abs(y).max())
    ox = oracle.quantize(X, oracle.ROWWISE)
    ow = oracle.quantize(W, oracle.TWO_D, with_codes_t=True)
    rng = np.random.default_rng(2)
    ms = np.concatenate([[0, 8191, 255, 256], rng.integers(0, 8192, 1500)])
    ns = np.concatenate([[0, 5119, 256, 255], rng.integers(0, 5120, 1500)])
    ref, t = oracle.gemm_entries(ox, ow, ms, ns)
    err = np.abs(y[ms, ns] - ref)
    lim = GEMM_TOL * t + 2.0 ** -8 * np.abs(ref)
    assert np.all(err <= lim), float(np.max(err / np.maximum(lim, 1e-300)))
    assert_gemm_every_entry(y, ox, ow, "bf16 fprop, every entry", rel=2.0 ** -8)


def test_half_width_tail_tiles_bf16():
    """17 x 16 tiles leave a last round of 16 tiles; with a BF16 output and
    no workspace they run as 32 half-width (256 x 128) workgroups over the
    whole K.  Those tiles
    (the last tile-row) are checked densely against the oracle within the GEMM
    tolerance plus BF16 rounding, the amax against the written values, and two
    runs bit for bit."""
    M, N, K = 17 * 256, 16 * 256, 1024
    qa, qb, x, w = _ops(M, N, K, 41)
    say("gemm bf16 half-width tail", (M, N, K))
    cb1, amax = nv.gemm_bf16(qa, qb, workspace=None)
    cb2, _ = nv.gemm_bf16(qa, qb, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(cb1, cb2)
    y = cb1.float().cpu().numpy().astype(np.float64)
    assert float(amax.cpu()[0]) == float(np.abs(y).max())
    ox, ow = oracle.quantize(x, oracle.ROWWISE), oracle.quantize(w, oracle.TWO_D)
    rng = np.random.default_rng(3)
    rows = np.concatenate([np.arange(16 * 256, M, 3), rng.integers(0, 16 * 256, 48)])
    cols = np.concatenate([np.arange(0, N, 29), [127, 128, N - 1]])
    ms, ns = np.meshgrid(rows, cols, indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    ref, t = oracle.gemm_entries(ox, ow, ms, ns)
    err = np.abs(y[ms, ns] - ref)
    lim = GEMM_TOL * t + 2.0 ** -8 * np.abs(ref)
    assert np.all(err <= lim), float(np.max(err / np.maximum(lim, 1e-300)))
    assert_gemm_every_entry(y, ox, ow, "half-width tail, every entry", rel=2.0 ** -8)


# Output layouts of the fast-path epilogue: 16-byte pieces of rows (4 FP32 /
# 8 BF16 values) when ldc and the base allow them, else 4- or 2-byte stores.
# Each case writes into a sentinel-filled buffer: the pitch padding past N
# and the bytes around the output must stay untouched.
def _ops_1d(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = inputs.normal(g, M, K, 1.0, 0.001, 50.0)
    w = inputs.normal(g, N, K, 0.02)
    return nv.quantize_1d(x.cuda()), nv.quantize_1d(w.cuda()), x, w


@pytest.mark.parametrize("case", [(272, 400, 512, 404, 0),    # 16-byte rows, padded pitch
                                  (272, 400, 512, 402, 0),    # pitch not a multiple of 4
                                  (272, 400, 512, 400, 1),    # base 4 bytes off 16
                                  (48, 80, 256, 84, 0)])      # one partial tile
def test_fp32_output_layouts(case):
    M, N, K, ldc, off = case
    qa, qb, x, w = _ops_1d(M, N, K, M + N + K + ldc)
    say("gemm fp32 layout", case)
    buf = torch.full((off + M * ldc + 64,), 7.0, device="cuda")
    nv.nvfp4_gemm(qa, qb, buf[off:], ldc)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    rows = got[off:off + M * ldc].reshape(M, ldc)
    ox, ow = oracle.quantize(x, oracle.ROWWISE), oracle.quantize(w, oracle.ROWWISE)
    c, t = oracle.gemm(ox, ow)
    err = np.abs(rows[:, :N].astype(np.float64) - c)
    assert np.all(err <= GEMM_TOL * t), float(np.max(err / np.maximum(GEMM_TOL * t, 1e-300)))
    assert np.all(rows[:, N:] == 7.0)
    assert np.all(got[:off] == 7.0) and np.all(got[off + M * ldc:] == 7.0)


@pytest.mark.parametrize("case", [(272, 304, 512, 312, 0),    # 16-byte rows, padded pitch
                                  (272, 304, 512, 306, 0),    # pitch not a multiple of 8
                                  (272, 304, 512, 304, 4),    # base 8 bytes off 16
                                  (48, 80, 256, 88, 0)])      # one partial tile
def test_bf16_output_layouts(case):
    M, N, K, ldc, off = case
    qa, qb, _, _ = _ops_1d(M, N, K, M + N + K + ldc)
    say("gemm bf16 layout", case)
    c32 = nv.gemm(qa, qb)
    sentinel = 0x7E57
    buf = torch.full((off + M * ldc + 64,), sentinel, dtype=torch.int16, device="cuda")
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm_bf16(qa, qb, buf[off:], ldc, amax)
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint16)
    rows = got[off:off + M * ldc].reshape(M, ldc)
    assert np.array_equal(rows[:, :N], rne_bf16_bits(c32.cpu().numpy()))
    assert np.all(rows[:, N:] == sentinel)
    assert np.all(got[:off] == sentinel) and np.all(got[off + M * ldc:] == sentinel)
    mag = (rows[:, :N] & 0x7FFF).astype(np.uint32) << 16
    assert float(amax.cpu()[0]) == float(mag.max().view(np.float32))
