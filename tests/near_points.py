"""Inputs whose scaled values v = z * r land within 16 binary32 patterns of
the points where the E2M1 decision changes: the midpoints between grid
values (round to nearest) and the grid values themselves (stochastic
rounding's carry boundaries).

The element scale r = 1/(E s_t) of a block depends on the tensor scale s_t
(from the given tensor amax) and the block's E4M3 code E.  For a random
tensor amax, every non-power-of-two code E gives its own r; for each target
point t the bf16 values z next to t/r are tried, and a hit is a z whose
fl(z * r) lies within 16 patterns of t (on either side).  Tensor amaxes are
drawn until every target has hits on both sides.  A block holds its largest
element b (chosen so that the block's code is E) and its hits; the rest of
the block is filled with smaller random values.  The CPU reference's own
block-scale and reciprocal functions decide E and r, so the construction is
checked against the reference by the test that uses it."""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle

TARGETS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                    0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
WINDOW = 16


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest bf16 (ties to even), as float32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32)


@dataclass
class Block:
    code: int              # intended E4M3 scale code
    bmax: float            # the block's largest magnitude (bf16)
    hits: list = field(default_factory=list)   # (z, target, delta_patterns)


@dataclass
class Tensor:
    amax: float            # the given tensor amax
    blocks: list


def _codes():
    """Scale codes whose value is not a power of two (so r is not one)."""
    out = []
    for c in range(1, 127):
        m = c & 7
        if (c >> 3) == 0:
            if m not in (1, 2, 4):
                out.append(c)
        elif m != 0:
            out.append(c)
    return np.array(out)


def _tensor_hits(amax_t: float, codes) -> Tensor:
    s_t = oracle.tensor_scale(amax_t)
    blocks = []
    for c in codes:
        E = oracle.e4m3_decode(int(c))
        r = np.float32(oracle.block_recip(int(c), s_t))
        if not np.isfinite(r) or r == 0:
            continue
        b = bf16_round(np.float32(6.0 * E * s_t * 1.004))
        if not (0 < b < 3e38) or oracle.block_scale(float(b), s_t) != c:
            continue
        z0 = (TARGETS.astype(np.float64) / float(r)).astype(np.float32)
        top = (z0.view(np.uint32) >> 16).astype(np.int64)
        cand = (top[:, None] + np.arange(-1, 3)[None, :]).astype(np.uint32) << 16
        z = cand.view(np.float32)
        v = z * r                                               # binary32 product
        d = v.view(np.uint32).astype(np.int64) - TARGETS.view(np.uint32).astype(np.int64)[:, None]
        ok = (np.abs(d) <= WINDOW) & (d != 0) & (z <= b) & (z > 0)
        blk = Block(int(c), float(b))
        for i, j in zip(*np.nonzero(ok)):
            blk.hits.append((float(z[i, j]), float(TARGETS[i]), int(d[i, j])))
        if blk.hits:
            blocks.append(blk)
    return Tensor(float(amax_t), blocks)


def _f32_near(x: float, k: int = 2) -> np.ndarray:
    b = int(np.float32(x).view(np.uint32))
    return np.arange(b - k, b + k + 1, dtype=np.int64).astype(np.uint32).view(np.float32)


def _solve(tgt: float, side: int, rng, codes, tries: int = 4000):
    """A tensor amax for which some bf16 z and non-power-of-two code E give
    fl(z * r) within WINDOW patterns of tgt on the given side.  Solved
    backwards: z and E drawn, then r, the block divisor E*s_t, s_t and the
    tensor amax each taken from the binary32 neighbours of the exact
    inverse; the reference's own functions confirm the solution."""
    t = np.float32(tgt)
    for _ in range(tries):
        c = int(rng.choice(codes))
        E = np.float32(oracle.e4m3_decode(c))
        z = bf16_round(np.float32(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-12, 12))))
        dv = side * int(rng.integers(1, WINDOW + 1))
        v_t = np.uint32(int(t.view(np.uint32)) + dv).view(np.float32)
        for r in _f32_near(float(v_t) / float(z), 3):
            if z * r != v_t:
                continue
            for d in _f32_near(1.0 / float(r)):
                if np.float32(1) / d != r:
                    continue
                for s_t in _f32_near(float(d) / float(E)):
                    if E * s_t != d:
                        continue
                    for a in _f32_near(2688.0 * float(s_t)):
                        if not (0 < a < 3e38) or oracle.tensor_scale(float(a)) != s_t:
                            continue
                        if np.float32(oracle.block_recip(c, float(s_t))) != r:
                            continue
                        return float(a)
    raise AssertionError(f"no solution for target {tgt} side {side}")


def find(seed: int = 0, per_side: int = 2):
    """Tensors (each with its own tensor amax) giving every target at least
    `per_side` hits below and above it (above 6 is saturation and is left
    out: the block maximum caps the scaled values there)."""
    rng = np.random.default_rng(seed)
    codes = _codes()
    need = {(float(t), s): per_side for t in TARGETS for s in (-1, 1)}
    need[(6.0, 1)] = 0
    out = []
    for key in sorted(need):
        while need[key] > 0:
            t = _tensor_hits(_solve(key[0], key[1], rng, codes), codes)
            for blk in t.blocks:
                for (_, tgt, d) in blk.hits:
                    k2 = (tgt, 1 if d > 0 else -1)
                    need[k2] = need.get(k2, 0) - 1
            out.append(t)
    return out


def rowwise_tensor(t: Tensor, rng, cols_blocks: int = 2) -> np.ndarray:
    """bf16 bit patterns [rows][16 * cols_blocks]: block i holds +-bmax, its
    hits (random signs) and random smaller values; rows padded with zeros."""
    blocks = []
    for blk in t.blocks:
        hits = [z for (z, _, _) in blk.hits]
        for s in range(0, max(len(hits), 1), 15):
            vals = np.zeros(16, np.float32)
            vals[0] = blk.bmax
            part = hits[s:s + 15]
            vals[1:1 + len(part)] = part
            fill = 15 - len(part)
            if fill:
                vals[1 + len(part):] = bf16_round(rng.uniform(0, blk.bmax, fill).astype(np.float32))
            rng.shuffle(vals)
            vals *= rng.choice(np.float32([-1, 1]), 16)
            blocks.append(vals)
    nb = len(blocks)
    per_row = cols_blocks
    rows = -(-nb // per_row)
    rows = -(-rows // 16) * 16
    x = np.zeros((rows * per_row, 16), np.float32)
    x[:nb] = np.stack(blocks)
    return bf16_round(x.reshape(rows, 16 * per_row)).view(np.uint32).__rshift__(16).astype(np.uint16)


def tiles_2d(t: Tensor, rng) -> np.ndarray:
    """bf16 bit patterns [16 * tiles][16]: one 16x16 tile per block (every
    tile shares one scale code), hits placed in it, the rest random."""
    tiles = []
    for blk in t.blocks:
        vals = bf16_round(rng.uniform(0, blk.bmax, 256).astype(np.float32))
        vals[0] = blk.bmax
        hits = [z for (z, _, _) in blk.hits][:255]
        vals[1:1 + len(hits)] = hits
        rng.shuffle(vals)
        vals *= rng.choice(np.float32([-1, 1]), 256)
        tiles.append(vals.reshape(16, 16))
    x = np.concatenate(tiles, axis=0)
    return bf16_round(x).view(np.uint32).__rshift__(16).astype(np.uint16)


def scaled_values(x_bits: np.ndarray, amax_t: float, scales: np.ndarray, blk_rows: int):
    """v = z * r of every element of a rowwise (blk_rows 1) or 2D (16)
    operand, with r from the reference's block scale codes."""
    s_t = oracle.tensor_scale(amax_t)
    z = (x_bits.astype(np.uint32) << 16).view(np.float32)
    R, C = z.shape
    sc = np.repeat(np.repeat(scales, blk_rows, axis=0), 16, axis=1)[:R, :C]
    rtab = np.array([oracle.block_recip(c, s_t) if c else 0.0 for c in range(127)], np.float32)
    return z * rtab[sc]


def window_coverage(v: np.ndarray):
    """{(target, side): count} of scaled values within WINDOW patterns of a target."""
    a = np.abs(v.ravel()).view(np.uint32).astype(np.int64)
    cov = {}
    for t in TARGETS:
        d = a - int(np.float32(t).view(np.uint32))
        for side in (-1, 1):
            m = (d * side > 0) & (np.abs(d) <= WINDOW)
            cov[(float(t), side)] = int(m.sum())
    return cov
