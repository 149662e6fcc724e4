"""Helpers shared by the GPU parity tests: move seeded host inputs to the
device, run the HIP path, and compare its outputs with the CPU oracle's."""
from __future__ import annotations

import contextlib
import math
import sys

import numpy as np
import torch

import oracle
import bit_microscaled_numerics_amd as nv

# GEMM tolerance: |C_gpu - C_exact| <= GEMM_TOL * sum_k |a_dec * b_dec| per element
GEMM_TOL = 1e-5


def say(*msg):
    """Name the case before each GPU step, flushed, so a fault names it."""
    print("[case]", *msg, file=sys.stderr, flush=True)


def f32_bits(x: float) -> int:
    return int(np.float32(x).view(np.uint32))


def dev_scalar(t: torch.Tensor) -> float:
    return float(t.cpu().numpy()[0])


def assert_operand_equal(g: nv.NVFP4Tensor, o: oracle.Operand, name: str = ""):
    gc = g.codes.cpu().numpy()
    gs = g.scales.cpu().numpy()
    assert gc.shape == o.codes.shape, name
    assert gs.shape == o.scales.shape, name
    assert f32_bits(dev_scalar(g.amax)) == f32_bits(o.amax), (name, dev_scalar(g.amax), o.amax)
    assert f32_bits(dev_scalar(g.tensor_scale)) == f32_bits(o.tensor_scale), name
    bad_s = np.argwhere(gs != o.scales)
    assert bad_s.size == 0, f"{name}: {len(bad_s)} scale mismatches, first {bad_s[:4].tolist()}"
    bad_c = np.argwhere(gc != o.codes)
    assert bad_c.size == 0, (f"{name}: {len(bad_c)} code-byte mismatches, first "
                             f"{bad_c[:4].tolist()} gpu={gc[tuple(bad_c[0])]:#04x} "
                             f"oracle={o.codes[tuple(bad_c[0])]:#04x}")
    if o.codes_t is not None:
        assert g.codes_t is not None
        assert np.array_equal(g.codes_t.cpu().numpy(), o.codes_t), f"{name}: codes_t"
    if g.scales_t is not None:  # 2D operand: the scale matrix transposed
        assert np.array_equal(g.scales_t.cpu().numpy(), o.scales.T), f"{name}: scales_t"


def assert_gemm_close(c_gpu: np.ndarray, c_ref: np.ndarray, t_ref: np.ndarray, name: str = ""):
    err = np.abs(c_gpu.astype(np.float64) - c_ref)
    lim = GEMM_TOL * t_ref
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{name}: {len(bad)} entries beyond tolerance; first "
                           f"{bad[:3].tolist()} err={err[tuple(bad[0])]:.3e} "
                           f"lim={lim[tuple(bad[0])]:.3e}")
    return float(np.max(err / np.maximum(t_ref, 1e-300)))


def assert_gemm_every_entry(c_gpu: np.ndarray, oa, ob, name: str = "", rel: float = 0.0):
    """Every entry of a GPU product against the oracle's float64 form (its own
    error, about K * 2^-53 * T, is far inside the tolerance); rel adds a
    relative allowance (2^-8 for a BF16 output's rounding)."""
    ref, t = oracle.gemm_f64(oa, ob)
    err = np.abs(c_gpu.astype(np.float64) - ref)
    lim = GEMM_TOL * t + rel * np.abs(ref)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{name}: {len(bad)} of {err.size} entries beyond tolerance; first "
                           f"{bad[:3].tolist()} err={err[tuple(bad[0])]:.3e} "
                           f"lim={lim[tuple(bad[0])]:.3e}")


# ---------------------------------------------------------------- guard bands
GUARD_BYTES = 4096
GUARD_FILL = 0xA5


class GuardBands:
    """A replacement for the binding's output allocator: every buffer sits
    inside a larger allocation with GUARD_BYTES of a sentinel byte on both
    sides, so a kernel that writes past either end of an output is caught
    (an exact-size torch.empty buffer would let such a write land silently in
    whatever the caching allocator put next to it)."""

    def __init__(self):
        self.bufs = []

    def empty(self, *shape, dtype, device):
        item = torch.empty(0, dtype=dtype).element_size()
        n = math.prod(shape) * item
        raw = torch.empty(n + 2 * GUARD_BYTES, dtype=torch.uint8, device=device)
        raw.fill_(GUARD_FILL)
        self.bufs.append((raw, n))
        return raw[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(*shape)

    def check(self):
        torch.cuda.synchronize()
        for raw, n in self.bufs:
            for part in (raw[:GUARD_BYTES], raw[GUARD_BYTES + n:]):
                bad = torch.nonzero(part != GUARD_FILL)
                assert bad.numel() == 0, (f"write outside an output buffer of {n} bytes: "
                                          f"{bad.numel()} guard bytes changed")
        self.bufs.clear()


@contextlib.contextmanager
def guard_bands():
    """Route the binding's output allocations through GuardBands for the
    duration, then check every guard."""
    g = GuardBands()
    saved = nv._empty
    nv._empty = g.empty
    try:
        yield g
    finally:
        nv._empty = saved
    g.check()
