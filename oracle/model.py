"""A second, pure-numpy model of the NVFP4 quantizer (TEST INFRASTRUCTURE).

Written independently of ``nvfp4_oracle.c`` in a different style: vectorised
numpy float32 arithmetic, the E4M3 encoder from frexp/rint instead of a table
bisection, the E2M1 rounding from midpoint thresholds instead of a nearest-
value search, and Philox in numpy uint64.  Used on tiny tensors only, where it
must agree byte for byte with the C oracle.  Readings as in the C oracle.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], F32)


# ---------------------------------------------------------------- Philox4x32-10
def philox(ctr: np.ndarray, key0: int, key1: int) -> np.ndarray:
    """ctr: uint64 array [n][4] holding 32-bit words -> [n][4] outputs."""
    M = np.uint64(0xFFFFFFFF)
    c = ctr.astype(np.uint64) & M
    k0, k1 = np.uint64(key0 & 0xFFFFFFFF), np.uint64(key1 & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(0x9E3779B9)) & M
            k1 = (k1 + np.uint64(0xBB67AE85)) & M
        p0 = np.uint64(0xD2511F53) * c[:, 0]
        p1 = np.uint64(0xCD9E8D57) * c[:, 2]
        c = np.stack([((p1 >> np.uint64(32)) ^ c[:, 1] ^ k0) & M, p1 & M,
                      ((p0 >> np.uint64(32)) ^ c[:, 3] ^ k1) & M, p0 & M], axis=1)
    return c


def sr_bits(seed: int, stream_id: int, n: np.ndarray) -> np.ndarray:
    n = n.astype(np.uint64)
    g = n >> np.uint64(3)
    ctr = np.stack([g & np.uint64(0xFFFFFFFF), g >> np.uint64(32),
                    np.full_like(g, stream_id), np.zeros_like(g)], axis=1)
    out = philox(ctr, seed & 0xFFFFFFFF, seed >> 32)
    word = out[np.arange(n.size), ((n & np.uint64(7)) >> np.uint64(1)).astype(np.int64)]
    half = (n & np.uint64(1)) * np.uint64(16)
    return ((word >> half) & np.uint64(0xFFFF)).astype(np.uint16)


def rht_signs(seed: int) -> int:
    out = philox(np.array([[0, 0, 0, 1]], np.uint64), seed & 0xFFFFFFFF, seed >> 32)
    return int(out[0, 0] & np.uint64(0xFFFF))


# ---------------------------------------------------------------- formats
def e4m3_value(code: np.ndarray) -> np.ndarray:
    code = code.astype(np.int64)
    e, m = (code >> 3) & 15, code & 7
    return np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e - 7)).astype(F32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Non-negative float32 -> E4M3FN code, RNE, saturating at 448."""
    x = np.asarray(x, F32).astype(np.float64)
    _, ex = np.frexp(np.where(x > 0, x, 1.0))       # x = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                      # unbiased exponent, clamped at min normal
    step = np.ldexp(1.0, e - 3)                      # spacing of E4M3 values at that exponent
    q = np.rint(x / step)                            # exact: x/step is a power-of-two scaling
    val = q * step
    val = np.minimum(val, 448.0)
    val = np.where(x > 0, val, 0.0)
    # value -> code
    _, vex = np.frexp(np.where(val > 0, val, 1.0))
    ve = vex - 1
    normal = val >= 2.0 ** -6
    code_n = ((ve + 7) << 3) | (np.rint(val / np.ldexp(1.0, ve - 3)).astype(np.int64) - 8)
    code_s = np.rint(val / 2.0 ** -9).astype(np.int64)
    return np.where(normal, code_n, code_s).astype(np.uint8)


# thresholds between consecutive E2M1 magnitudes and whether the midpoint
# itself rounds up (ties go to the even index)
_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], F32)
_MID_UP = np.array([False, True, False, True, False, True, False])


def e2m1_rtn(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, F32)
    a = np.abs(v)
    idx = np.zeros(a.shape, np.int64)
    for t, up in zip(_MID, _MID_UP):
        idx += (a >= t) if up else (a > t)
    return (np.signbit(v).astype(np.int64) * 8 + idx).astype(np.uint8)


def e2m1_sr(v: np.ndarray, u16: np.ndarray) -> np.ndarray:
    v = np.asarray(v, F32)
    a = np.minimum(np.abs(v), F32(6.0))
    lo = np.searchsorted(E2M1_MAG, a, side="right") - 1
    hi = np.minimum(lo + 1, 7)
    glo, ghi = E2M1_MAG[lo], E2M1_MAG[hi]
    on_grid = glo == a
    gap = np.where(on_grid, F32(1.0), ghi - glo)
    p = ((a - glo) / gap).astype(F32)
    up = (~on_grid) & (u16.astype(F32) < p * F32(65536.0))
    idx = np.where(up, hi, lo)
    return (np.signbit(v).astype(np.int64) * 8 + idx).astype(np.uint8)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, np.int64)
    return np.where(code & 8, -1.0, 1.0).astype(F32) * E2M1_MAG[code & 7]


# ---------------------------------------------------------------- RHT
def rht_rows(z: np.ndarray, signs: int) -> np.ndarray:
    """Apply 1/4 H16 D to every 16-group along the last axis (float32)."""
    z = np.asarray(z, F32)
    s = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(16)], F32)
    w = (z.reshape(z.shape[:-1] + (-1, 16)) * s).astype(F32)
    h = 1
    while h < 16:
        w = w.reshape(w.shape[:-1] + (16 // (2 * h), 2, h))
        a, b = w[..., 0, :], w[..., 1, :]
        w = np.stack([a + b, a - b], axis=-2).astype(F32)
        w = w.reshape(w.shape[:-3] + (16,))
        h *= 2
    return (w * F32(0.25)).astype(F32).reshape(z.shape)


# ---------------------------------------------------------------- quantizer
def quantize(x_bits: np.ndarray, mode: int, rht_seed=None, sr_seed=None, stream_id=0):
    """Returns (codes uint8 [I][K] unpacked, scales, s_t, amax)."""
    x = (x_bits.astype(np.uint32) << 16).view(F32)
    z = x.T.copy() if mode == 1 else x.copy()
    I, K = z.shape
    if rht_seed is not None:
        z = rht_rows(z, rht_signs(rht_seed))
    amax = F32(np.max(np.abs(z))) if z.size else F32(0)
    s_t = F32(amax / F32(2688.0)) if amax > 0 else F32(1.0)
    t6 = F32(F32(6.0) * s_t)
    if mode == 2:
        blocks = np.abs(z).reshape(I // 16, 16, K // 16, 16).max(axis=(1, 3))
        amax_b = np.repeat(np.repeat(blocks, 16, axis=0), 16, axis=1)
    else:
        blocks = np.abs(z).reshape(I, K // 16, 16).max(axis=2)
        amax_b = np.repeat(blocks, 16, axis=1)
    E = e4m3_encode((blocks / t6).astype(F32))
    Eel = e4m3_encode((amax_b / t6).astype(F32))
    d = (e4m3_value(Eel) * s_t).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (F32(1.0) / d).astype(F32)
        v = (z * r).astype(F32)
    if sr_seed is not None:
        n = np.arange(I * K, dtype=np.uint64).reshape(I, K)
        u = sr_bits(sr_seed, stream_id, n.ravel()).reshape(I, K)
        codes = e2m1_sr(v, u)
    else:
        codes = e2m1_rtn(v)
    zero = Eel == 0
    codes = np.where(zero, np.signbit(z).astype(np.uint8) * 8, codes).astype(np.uint8)
    return codes, E, s_t, amax


def pack(codes: np.ndarray) -> np.ndarray:
    """[I][K] nibbles -> [I][K/2] bytes, even k in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    p = packed.astype(np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


# ---------------------------------------------------------------- MXFP4
def e8m0_encode(amax: np.ndarray) -> np.ndarray:
    """E8M0 byte e + 127 with e = ceil(log2(amax / 6)), clamped to [-127, 127];
    amax == 0 -> 0.  amax / 6 is formed in float64, where it is exact enough
    for the ceiling (a float32 amax has 24 significant bits); frexp gives
    amax / 6 = f * 2^x with f in [0.5, 1), so ceil(log2) is x - 1 when f is
    exactly 0.5 and x otherwise."""
    a = np.asarray(amax, np.float64)
    f, x = np.frexp(np.where(a > 0, a / 6.0, 1.0))
    e = np.where(f == 0.5, x - 1, x)
    e = np.clip(e, -127, 127)
    return np.where(a > 0, e + 127, 0).astype(np.uint8)


def mx_quantize(x_bits: np.ndarray, sr_seed=None, stream_id=0):
    """Rowwise MXFP4 of bf16 bits [rows][cols] -> (codes uint8 [rows][cols]
    unpacked, scales uint8 [rows][cols/32])."""
    z = (x_bits.astype(np.uint32) << 16).view(F32)
    R, K = z.shape
    amax_b = np.abs(z).reshape(R, K // 32, 32).max(axis=2)
    sc = e8m0_encode(amax_b)
    inv = np.ldexp(F32(1.0), 127 - sc.astype(np.int32)).astype(F32)   # 2^-e
    v = (z * np.repeat(inv, 32, axis=1)).astype(F32)
    if sr_seed is not None:
        n = np.arange(R * K, dtype=np.uint64)
        codes = e2m1_sr(v, sr_bits(sr_seed, stream_id, n).reshape(R, K))
    else:
        codes = e2m1_rtn(v)
    return codes, sc
