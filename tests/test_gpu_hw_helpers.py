"""The NVFP4 kernels' helpers that take their decisions from gfx950 hardware
converts, run on the GPU over whole ranges of binary32 inputs and compared
with the CPU reference's bit-level definitions:

  * the E4M3 block-scale encode (FP8 convert after a clamp to 448) on every
    binary32 in [0, 448] and a sweep above it ("NVFP4 Trains with Precision
    of 16-Bit and Speed and Efficiency of 4-Bit", E4M3 scale factors:
    round to nearest, saturating);
  * the E2M1 round-to-nearest-even encode (FP4 convert) on every binary32 in
    [-8, 8] and a sweep beyond ("Pretraining Large Language Models with
    NVFP4", format paragraph: values 0, 0.5 ... 6);
  * the E2M1 stochastic-rounding encode (software decision, FP4 convert of
    the chosen grid value) near every decision point with all 65536 random
    values, and on a strided sweep (NVIDIA blog, stochastic-rounding
    section);
  * the block-scale step (reciprocal multiply with an exact-division
    fallback near E4M3 rounding points, and always below amax ~1.3e-36)
    against the correctly rounded quotient, for many tensor amaxes, every
    E4M3 midpoint +-64 patterns, and random block amaxes;
  * the GEMM's operand decode (FP4 -> FP16 convert scaled by 2^floor(log2
    E), times E's mantissa) for every scale code and every code at every
    nibble position, by its ALU, table and pair forms (the pair form takes
    the code from either byte of either half of a scale dword).

The helpers are compiled from the kernels' own headers into a test-only
library (tests/devhelpers)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import devtest
from parity import say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26
E2M1 = np.array([oracle.e2m1_decode(c) for c in range(16)], np.float32)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _unpack(packed: np.ndarray) -> np.ndarray:
    out = np.empty(packed.size * 2, np.uint8)
    out[0::2] = packed & 0xF
    out[1::2] = packed >> 4
    return out


def _first_bad(got, want, inputs):
    bad = np.flatnonzero(got != want)
    if bad.size:
        i = bad[0]
        x = inputs[i]
        raise AssertionError(f"{bad.size} mismatches; first input {x!r} "
                             f"({np.float32(x).view(np.uint32):#010x}) gpu={got[i]} reference={want[i]}")


def _e4m3_gpu(x: torch.Tensor) -> np.ndarray:
    out = torch.empty(x.numel(), dtype=torch.uint8, device="cuda")
    assert devtest.load().devtest_e4m3_code(x.data_ptr(), out.data_ptr(), x.numel(), _stream()) == 0
    return out.cpu().numpy()


def test_e4m3_encode_every_binary32_to_448():
    hi = int(np.float32(448.0).view(np.uint32))
    for start in range(0, hi + 1, CHUNK):
        n = min(CHUNK, hi + 1 - start)
        say("e4m3 encode patterns", hex(start), n)
        x = torch.arange(start, start + n, dtype=torch.int32, device="cuda").view(torch.float32)
        got = _e4m3_gpu(x)
        xs = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
        _first_bad(got, oracle.e4m3_encode(xs), xs)


def test_e4m3_encode_saturates_above_448():
    lo, hi = int(np.float32(448.0).view(np.uint32)), int(np.float32(3.0e38).view(np.uint32))
    xs = np.arange(lo, hi, 4099, dtype=np.uint32).view(np.float32)
    say("e4m3 encode above 448", xs.size)
    got = _e4m3_gpu(torch.from_numpy(xs).cuda())
    assert np.all(got == 0x7E)
    _first_bad(got, oracle.e4m3_encode(xs), xs)


def _rtn_gpu(v: torch.Tensor) -> np.ndarray:
    out = torch.empty(v.numel() // 2, dtype=torch.uint8, device="cuda")
    assert devtest.load().devtest_encode_rtn(v.data_ptr(), out.data_ptr(), v.numel(), _stream()) == 0
    return _unpack(out.cpu().numpy())


@pytest.mark.parametrize("sign", [0, 1])
def test_e2m1_rtn_every_binary32_to_8(sign):
    hi = int(np.float32(8.0).view(np.uint32))
    end = (hi + 1 + 7) // 8 * 8
    for start in range(0, end, CHUNK):
        n = min(CHUNK, end - start)
        say("e2m1 rtn patterns", sign, hex(start), n)
        v = torch.arange(start, start + n, dtype=torch.int32, device="cuda").view(torch.float32)
        vs = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
        if sign:   # negation flips only the sign bit (-0 included)
            v, vs = -v, -vs
        got = _rtn_gpu(v)
        _first_bad(got, oracle.e2m1_rtn(vs), vs)


def test_e2m1_rtn_saturates_beyond_8():
    lo, hi = int(np.float32(8.0).view(np.uint32)), int(np.float32(3.0e38).view(np.uint32))
    vs = np.arange(lo, hi, 4097, dtype=np.uint32).view(np.float32)
    vs = np.concatenate([vs, -vs])[: (2 * vs.size) // 8 * 8]
    say("e2m1 rtn beyond 8", vs.size)
    got = _rtn_gpu(torch.from_numpy(vs).cuda())
    _first_bad(got, oracle.e2m1_rtn(vs), vs)
    assert np.all((got & 7) == 7)


def _sr_check(v: np.ndarray, u: np.ndarray):
    n = v.size // 8 * 8
    v, u = v[:n], u[:n]
    out = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    vd, ud = torch.from_numpy(v).cuda(), torch.from_numpy(u.view(np.int16)).cuda()
    assert devtest.load().devtest_encode_sr(vd.data_ptr(), ud.data_ptr(), out.data_ptr(), n,
                                            _stream()) == 0
    got = _unpack(out.cpu().numpy())
    _first_bad(got, oracle.e2m1_sr(v, u), v)


def test_e2m1_sr_near_decision_points_all_random_values():
    v = devtest.sr_near_points()
    u = np.arange(65536, dtype=np.uint16)
    say("e2m1 sr near points", v.size)
    for i in range(0, v.size, 256):
        vv = v[i:i + 256]
        _sr_check(np.repeat(vv, u.size), np.tile(u, vv.size))


def test_e2m1_sr_strided_values():
    v = devtest.sr_strided_values(4099)
    u = np.arange(0, 65536, 97, dtype=np.uint16)
    say("e2m1 sr strided", v.size)
    for i in range(0, v.size, 65536):
        vv = v[i:i + 65536]
        _sr_check(np.repeat(vv, u.size), np.tile(u, vv.size))


def _e4m3_values() -> np.ndarray:
    return np.array([oracle.e4m3_decode(c) for c in range(127)], np.float64)


AMAXES = [2688.0, 784.0 * 2.0 ** -3, 1.0, 448.0, 3.0e4, 6.1e-5, 1.7e-20, 2.0 ** -100,
          1.0e-37, 3.0e-39] + list(np.random.default_rng(11).uniform(0.5, 2.0, 6)
                                   * 2.0 ** np.random.default_rng(12).integers(-40, 40, 6))


@pytest.mark.parametrize("amax_t", AMAXES)
def test_block_scale_step(amax_t):
    """Scale code of the correctly rounded amax_b / (6 s_t) and reciprocal
    1 / (E s_t), for block amaxes within 64 patterns of every point where
    the code changes (E4M3 midpoints times 6 s_t) and random ones; below an
    amax of about 1.3e-36 the kernels' 1/(6 s_t) overflows and every block
    takes the division."""
    amax_t = float(np.float32(amax_t))
    s_t = oracle.tensor_scale(amax_t)
    t6 = np.float32(6.0) * np.float32(s_t)
    vals = _e4m3_values()
    pts = np.concatenate([(vals[:-1] + vals[1:]) / 2, vals]) * float(t6)
    pts = pts[(pts > 1e-45) & (pts < 3e38)]
    base = pts.astype(np.float32).view(np.uint32).astype(np.int64)
    cand = (base[:, None] + np.arange(-64, 65)[None, :]).ravel()
    cand = cand[(cand > 0) & (cand < 0x7F800000)].astype(np.uint32).view(np.float32)
    rng = np.random.default_rng(int(np.float32(amax_t).view(np.uint32)))
    rnd = (amax_t * 2.0 ** rng.uniform(-30, 0, 20000)).astype(np.float32)
    amax_b = np.concatenate([cand, rnd, np.float32([0.0, amax_t])]).astype(np.float32)
    say("block scale", amax_t, amax_b.size)
    bd = torch.from_numpy(amax_b).cuda()
    code = torch.empty(amax_b.size, dtype=torch.uint8, device="cuda")
    r = torch.empty(amax_b.size, dtype=torch.float32, device="cuda")
    assert devtest.load().devtest_block_scale(bd.data_ptr(), amax_b.size, ctypes.c_float(amax_t),
                                              code.data_ptr(), r.data_ptr(), _stream()) == 0
    got_c, got_r = code.cpu().numpy(), r.cpu().numpy()
    want_c = np.array([oracle.block_scale(float(a), s_t) for a in amax_b], np.uint8)
    _first_bad(got_c, want_c, amax_b)
    nz = want_c != 0
    want_r = np.array([oracle.block_recip(int(c), s_t) for c in want_c[nz]], np.float32)
    _first_bad(got_r[nz].view(np.uint32), want_r.view(np.uint32), amax_b[nz])
    if amax_t < 1.3e-36:
        with np.errstate(over="ignore"):                # the division path is the one taken
            assert not np.isfinite(np.float32(1.0) / t6)


def test_gemm_operand_decode_every_scale_and_code():
    words = [0x11111111 * j for j in range(16)] + [0x76543210, 0xFEDCBA98, 0x89ABCDEF, 0x01234567]
    w = np.array([wd for _ in range(127) for wd in words], np.uint32)
    sc = np.repeat(np.arange(127, dtype=np.uint8), len(words))
    say("gemm decode", w.size)
    wd, sd = torch.from_numpy(w.view(np.int32)).cuda(), torch.from_numpy(sc).cuda()
    alu = torch.empty(w.size * 8, dtype=torch.int16, device="cuda")
    lut = torch.empty(w.size * 8, dtype=torch.int16, device="cuda")
    pair = torch.empty(w.size * 8, dtype=torch.int16, device="cuda")
    assert devtest.load().devtest_gemm_decode(wd.data_ptr(), sd.data_ptr(), alu.data_ptr(),
                                              lut.data_ptr(), pair.data_ptr(), w.size,
                                              _stream()) == 0
    nib = ((w[:, None] >> (4 * np.arange(8, dtype=np.uint32))[None, :]) & 0xF).astype(np.uint8)
    E = np.array([oracle.e4m3_decode(c) for c in range(127)], np.float32)
    want = (E2M1[nib] * E[sc][:, None]).astype(np.float16).ravel()
    assert np.array_equal(want.astype(np.float32), E2M1[nib].ravel() * np.repeat(E[sc], 8))
    for name, got in (("alu", alu), ("table", lut), ("pair", pair)):
        g = got.cpu().numpy().view(np.float16)
        bad = np.flatnonzero(g != want)     # +-0 compare equal: a zero scale may give either sign
        assert bad.size == 0, (name, bad.size, int(sc[bad[0] // 8]), hex(int(w[bad[0] // 8])),
                               float(g[bad[0]]), float(want[bad[0]]))
