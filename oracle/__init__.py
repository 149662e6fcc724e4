"""CPU oracle for NVFP4 quantization and the NVFP4-linear GEMM.

TEST INFRASTRUCTURE ONLY: the plain, slow reference the GPU library is checked
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it.  It shares no code with the HIP library and imports nothing
from it.  The arithmetic lives in ``nvfp4_oracle.c`` (binary32, no FMA
contraction, exact int64 GEMM; ``gemm_f64`` is its float64 form for whole
full-size products, a float64 library matmul of the exactly decoded operands)
and, for the MXFP4 comparison format,
``mxfp4_oracle.c``; this module is ctypes marshalling over numpy arrays.
``oracle.model`` is a second, pure-numpy model for tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# NVFP4_ORACLE_LIB selects another build of the same sources (the sanitizer
# build the tests run the oracle's own suite against).
_LIB_PATH = os.environ.get("NVFP4_ORACLE_LIB", os.path.join(_HERE, "liboracle.so"))
_lib = None

ROWWISE, COLWISE, TWO_D = 0, 1, 2

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64, _u64, _u32, _i32, _f32 = (ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                ctypes.c_int32, ctypes.c_float)

_OPERAND = [_u8p, _i64, _u8p, _i64, _i64, _i32, _f32, _i64]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_philox4x32_10": (None, [_u32p, _u32p, _u32p]),
        "orc_sr_bits": (ctypes.c_uint16, [_u64, _u32, _u64]),
        "orc_sr_bits_array": (None, [_u64, _u32, _u64, _i64, _u16p]),
        "orc_rht_signs": (ctypes.c_uint16, [_u64]),
        "orc_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "orc_e4m3_encode_array": (None, [_f32p, _i64, _u8p]),
        "orc_e2m1_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "orc_e2m1_rtn": (ctypes.c_uint8, [ctypes.c_float]),
        "orc_e2m1_rtn_array": (None, [_f32p, _i64, _u8p]),
        "orc_e2m1_sr": (ctypes.c_uint8, [ctypes.c_float, ctypes.c_uint16]),
        "orc_e2m1_sr_array": (None, [_f32p, _u16p, _i64, _u8p]),
        "orc_rht16": (None, [_f32p, ctypes.c_uint16, _f32p]),
        "orc_e8m0_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "orc_e8m0_encode_array": (None, [_f32p, _i64, _u8p]),
        "orc_e8m0_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "orc_mx_quantize": (ctypes.c_int, [_u16p, _i64, _i64, ctypes.c_int, _u64, _u32, _u8p, _u8p]),
        "orc_mx_dequantize": (None, [_u8p, _u8p, _i64, _i64, _f32p]),
        "orc_mx_gemm": (ctypes.c_int, [_u8p, _u8p, _i64, _u8p, _u8p, _i64, _i64, _f64p, _f64p]),
        "orc_mx_decode_exact": (ctypes.c_int, [_u8p, _u8p, _i64, _i64, _f64p]),
        "orc_mx_gemm_entries": (ctypes.c_int, [_u8p, _u8p, _u8p, _u8p, _i64, _i64p, _i64p, _i64,
                                               _f64p, _f64p]),
        "orc_amax": (ctypes.c_float, [_u16p, _i64, _i64]),
        "orc_amax_rht": (ctypes.c_float, [_u16p, _i64, _i64, _u64]),
        "orc_tensor_scale": (ctypes.c_float, [ctypes.c_float]),
        "orc_block_scale": (ctypes.c_uint8, [ctypes.c_float, ctypes.c_float]),
        "orc_block_recip": (ctypes.c_float, [ctypes.c_uint8, ctypes.c_float]),
        "orc_quantize": (ctypes.c_int, [_u16p, _i64, _i64, ctypes.c_int, ctypes.c_int, _u64,
                                        ctypes.c_int, _u64, _u32, ctypes.c_int, _f32p,
                                        _u8p, _u8p, _u8p, _f32p]),
        "orc_dequantize": (None, [_u8p, _i64, _u8p, _i64, _i64, _i32, _f32, _i64, _i64, _f32p]),
        "orc_gemm": (ctypes.c_int, _OPERAND + _OPERAND + [_i64, _f64p, _f64p]),
        "orc_decode_exact": (ctypes.c_int, _OPERAND + [_i64, _f64p]),
        "orc_gemm_entries": (ctypes.c_int, _OPERAND + _OPERAND + [_i64, _i64p, _i64p, _i64,
                                                                  _f64p, _f64p]),
        "orc_num_threads": (ctypes.c_int, []),
        "orc_set_num_threads": (None, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray, typ):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(typ)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the reference's parallel loops from now on (timing only)."""
    _load().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------- scalars
def philox4x32_10(ctr, key):
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib.orc_philox4x32_10(c, k, o)
    return [int(o[i]) for i in range(4)]


def sr_bits(seed: int, stream_id: int, n0: int, count: int) -> np.ndarray:
    out = np.empty(count, np.uint16)
    _load().orc_sr_bits_array(seed, stream_id, n0, count, _ptr(out, _u16p))
    return out


def rht_signs(seed: int) -> int:
    return int(_load().orc_rht_signs(seed))


def e4m3_decode(code: int) -> float:
    return float(_load().orc_e4m3_decode(code))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(x, _f32p), x.size, _ptr(out, _u8p))
    return out


def e2m1_decode(code: int) -> float:
    return float(_load().orc_e2m1_decode(code))


def e2m1_rtn(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e2m1_rtn_array(_ptr(v, _f32p), v.size, _ptr(out, _u8p))
    return out


def e2m1_sr(v: np.ndarray, u16: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, np.float32)
    u16 = np.ascontiguousarray(np.broadcast_to(u16, v.shape), np.uint16)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e2m1_sr_array(_ptr(v, _f32p), _ptr(u16, _u16p), v.size, _ptr(out, _u8p))
    return out


def rht16(x: np.ndarray, signs: int) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).reshape(16)
    out = np.empty(16, np.float32)
    _load().orc_rht16(_ptr(x, _f32p), signs, _ptr(out, _f32p))
    return out


def tensor_scale(amax: float) -> float:
    return float(_load().orc_tensor_scale(amax))


def block_scale(amax_b: float, s_t: float) -> int:
    """E4M3 code of a block with largest magnitude amax_b in a tensor of scale s_t."""
    return int(_load().orc_block_scale(amax_b, s_t))


def block_recip(code: int, s_t: float) -> float:
    """Element scale 1 / (E * s_t) of a block with scale code E."""
    return float(_load().orc_block_recip(code, s_t))


# --------------------------------------------------------------------------- tensors
def _as_bf16_bits(x) -> np.ndarray:
    """Accept a numpy uint16 array of bf16 bit patterns or a torch bf16 tensor."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.bfloat16
    return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def amax(x) -> float:
    x = _as_bf16_bits(x)
    return float(_load().orc_amax(_ptr(x, _u16p), x.shape[0], x.shape[1]))


def amax_rht(x, rht_seed: int) -> float:
    x = _as_bf16_bits(x)
    return float(_load().orc_amax_rht(_ptr(x, _u16p), x.shape[0], x.shape[1], rht_seed))


@dataclass
class Operand:
    """A quantized GEMM operand, logically [rows][k], K-contiguous."""
    codes: np.ndarray          # uint8 [rows][ld_codes]
    scales: np.ndarray         # uint8, indexed (r // blk_rows) * ss_row + (k // 16) * ss_k
    ss_row: int
    ss_k: int
    blk_rows: int
    tensor_scale: float
    rows: int
    k: int
    amax: float = 0.0
    codes_t: np.ndarray | None = None   # 2D only: [k][rows/2], the same codes transposed

    @property
    def ld_codes(self) -> int:
        return self.codes.shape[1]

    def transposed(self) -> "Operand":
        """The 2D operand read as its transpose (Dgrad's B)."""
        assert self.blk_rows == 16 and self.codes_t is not None
        return Operand(self.codes_t, self.scales, self.ss_k, self.ss_row, 16,
                       self.tensor_scale, self.k, self.rows, self.amax, self.codes)


def quantize(x, mode: int, *, rht_seed: int | None = None, sr_seed: int | None = None,
             stream_id: int = 0, amax_given: float | None = None,
             with_codes_t: bool = False) -> Operand:
    """Quantize bf16 x [rows][cols] (the six steps: tensor amax, tensor scale,
    block amax, E4M3 block scale, E2M1 encode RTN/SR, optional RHT)."""
    x = _as_bf16_bits(x)
    rows, cols = x.shape
    I, K = (cols, rows) if mode == COLWISE else (rows, cols)
    codes = np.zeros((I, K // 2), np.uint8)
    codes_t = np.zeros((K, I // 2), np.uint8) if (mode == TWO_D and with_codes_t) else None
    if mode == TWO_D:
        scales = np.zeros((rows // 16, cols // 16), np.uint8)
    else:
        scales = np.zeros((I, K // 16), np.uint8)
    amax_io = np.array([0.0 if amax_given is None else amax_given], np.float32)
    s_t = np.zeros(1, np.float32)
    rc = _load().orc_quantize(
        _ptr(x, _u16p), rows, cols, mode,
        int(rht_seed is not None), 0 if rht_seed is None else rht_seed,
        int(sr_seed is not None), 0 if sr_seed is None else sr_seed, stream_id,
        int(amax_given is not None), _ptr(amax_io, _f32p),
        _ptr(codes, _u8p), _ptr(codes_t, _u8p) if codes_t is not None else None,
        _ptr(scales, _u8p), _ptr(s_t, _f32p))
    if rc != 0:
        raise ValueError(f"oracle quantize rejected the arguments (status {rc})")
    if mode == TWO_D:
        ss_row, ss_k, blk = cols // 16, 1, 16
    else:
        ss_row, ss_k, blk = K // 16, 1, 1
    return Operand(codes, scales, ss_row, ss_k, blk, float(s_t[0]), I, K,
                   float(amax_io[0]), codes_t)


def _operand_args(q: Operand):
    codes = np.ascontiguousarray(q.codes)
    scales = np.ascontiguousarray(q.scales)
    return ([_ptr(codes, _u8p), codes.shape[1], _ptr(scales, _u8p), q.ss_row, q.ss_k,
             q.blk_rows, q.tensor_scale, q.rows], (codes, scales))


def dequantize(q: Operand) -> np.ndarray:
    out = np.empty((q.rows, q.k), np.float32)
    args, _keep = _operand_args(q)
    _load().orc_dequantize(args[0], args[1], args[2], args[3], args[4], args[5], args[6],
                           q.rows, q.k, _ptr(out, _f32p))
    return out


def gemm(a: Operand, b: Operand, with_bound: bool = True):
    """C[m][n] = s_a*s_b*sum_k A[m,k]*B[n,k] (exact int64 sum, then double);
    also T = sum_k |A*B| when with_bound."""
    assert a.k == b.k
    c = np.empty((a.rows, b.rows), np.float64)
    t = np.empty((a.rows, b.rows), np.float64) if with_bound else None
    aa, _ka = _operand_args(a)
    bb, _kb = _operand_args(b)
    rc = _load().orc_gemm(*aa, *bb, a.k, _ptr(c, _f64p), _ptr(t, _f64p) if t is not None else None)
    if rc != 0:
        raise ValueError(f"oracle gemm rejected the arguments (status {rc})")
    return (c, t) if with_bound else c


def decode_exact(q: Operand) -> np.ndarray:
    """q * E of every element (without the tensor scale) as float64 [rows][k]
    (exact; zeros as +0)."""
    out = np.empty((q.rows, q.k), np.float64)
    args, _keep = _operand_args(q)
    rc = _load().orc_decode_exact(*args, q.k, _ptr(out, _f64p))
    if rc != 0:
        raise ValueError(f"oracle decode rejected the arguments (status {rc})")
    return out


def gemm_f64(a: Operand, b: Operand, with_bound: bool = True):
    """The GEMM of ``gemm`` through a float64 matrix product of the exactly
    decoded operands (the product is a library routine; summation error at
    most about K * 2^-53 * T), then times s_a * s_b; also T = sum_k |A*B|
    the same way when with_bound.  Fast enough for whole full-size products."""
    assert a.k == b.k
    da, db = decode_exact(a), decode_exact(b)
    s = float(np.float64(a.tensor_scale) * np.float64(b.tensor_scale))
    c = (da @ db.T) * s
    if not with_bound:
        return c
    np.abs(da, out=da)
    np.abs(db, out=db)
    t = (da @ db.T) * abs(s)
    return c, t


def gemm_entries(a: Operand, b: Operand, ms: np.ndarray, ns: np.ndarray):
    """The entries (ms[j], ns[j]) of the product, with their bounds T."""
    assert a.k == b.k
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    c = np.empty(ms.size, np.float64)
    t = np.empty(ms.size, np.float64)
    aa, _ka = _operand_args(a)
    bb, _kb = _operand_args(b)
    rc = _load().orc_gemm_entries(*aa, *bb, a.k, _ptr(ms, _i64p), _ptr(ns, _i64p), ms.size,
                                  _ptr(c, _f64p), _ptr(t, _f64p))
    if rc != 0:
        raise ValueError(f"oracle gemm rejected the arguments (status {rc})")
    return c, t


# ---------------------------------------------------------------------------
# MXFP4 (the comparison format): 32-element blocks along K, power-of-two E8M0
# block scale, no tensor scale ("Pretraining Large Language Models with
# NVFP4", summary page, format paragraph).  Arithmetic in mxfp4_oracle.c.
# ---------------------------------------------------------------------------
def e8m0_encode(amax: np.ndarray) -> np.ndarray:
    """E8M0 byte e + 127, e the smallest integer with amax <= 6 * 2^e (clamped)."""
    a = np.ascontiguousarray(np.asarray(amax, np.float32).ravel())
    out = np.empty(a.size, np.uint8)
    _load().orc_e8m0_encode_array(_ptr(a, _f32p), a.size, _ptr(out, _u8p))
    return out.reshape(np.shape(amax))


def e8m0_decode(code: int) -> float:
    return float(_load().orc_e8m0_decode(code))


@dataclass
class MXOperand:
    """An MXFP4 GEMM operand, logically [rows][k], K-contiguous."""
    codes: np.ndarray    # uint8 [rows][k/2], low nibble = even k
    scales: np.ndarray   # uint8 E8M0 [rows][k/32]
    rows: int
    k: int


def mx_quantize(x, *, sr_seed: int | None = None, stream_id: int = 0) -> MXOperand:
    """Rowwise MXFP4 quantization of bf16 x [rows][cols] (cols % 32 == 0)."""
    x = _as_bf16_bits(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    rc = _load().orc_mx_quantize(_ptr(x, _u16p), rows, cols, int(sr_seed is not None),
                                 0 if sr_seed is None else sr_seed, stream_id,
                                 _ptr(codes, _u8p), _ptr(scales, _u8p))
    if rc != 0:
        raise ValueError(f"oracle mx_quantize rejected the arguments (status {rc})")
    return MXOperand(codes, scales, rows, cols)


def mx_dequantize(q: MXOperand) -> np.ndarray:
    out = np.empty((q.rows, q.k), np.float32)
    codes, scales = np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales)
    _load().orc_mx_dequantize(_ptr(codes, _u8p), _ptr(scales, _u8p), q.rows, q.k, _ptr(out, _f32p))
    return out


def mx_gemm(a: MXOperand, b: MXOperand):
    """C[m][n] = sum_k A[m,k]*B[n,k] in float64 (exact products), and
    T = sum_k |A*B|."""
    assert a.k == b.k
    c = np.empty((a.rows, b.rows), np.float64)
    t = np.empty((a.rows, b.rows), np.float64)
    ac, as_ = np.ascontiguousarray(a.codes), np.ascontiguousarray(a.scales)
    bc, bs = np.ascontiguousarray(b.codes), np.ascontiguousarray(b.scales)
    rc = _load().orc_mx_gemm(_ptr(ac, _u8p), _ptr(as_, _u8p), a.rows, _ptr(bc, _u8p),
                             _ptr(bs, _u8p), b.rows, a.k, _ptr(c, _f64p), _ptr(t, _f64p))
    if rc != 0:
        raise ValueError(f"oracle mx_gemm rejected the arguments (status {rc})")
    return c, t


def mx_decode_exact(q: MXOperand) -> np.ndarray:
    """Every decoded MXFP4 value as float64 [rows][k] (exact)."""
    out = np.empty((q.rows, q.k), np.float64)
    codes, scales = np.ascontiguousarray(q.codes), np.ascontiguousarray(q.scales)
    rc = _load().orc_mx_decode_exact(_ptr(codes, _u8p), _ptr(scales, _u8p), q.rows, q.k,
                                     _ptr(out, _f64p))
    if rc != 0:
        raise ValueError(f"oracle mx decode rejected the arguments (status {rc})")
    return out


def mx_gemm_f64(a: MXOperand, b: MXOperand):
    """mx_gemm through one float64 library matmul of the exactly decoded
    operands (and T from their magnitudes): the same float64 arithmetic in
    another summation order, fast enough for whole full-size products."""
    assert a.k == b.k
    da, db = mx_decode_exact(a), mx_decode_exact(b)
    c = da @ db.T
    np.abs(da, out=da)
    np.abs(db, out=db)
    return c, da @ db.T


def mx_gemm_entries(a: MXOperand, b: MXOperand, ms: np.ndarray, ns: np.ndarray):
    assert a.k == b.k
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    c = np.empty(ms.size, np.float64)
    t = np.empty(ms.size, np.float64)
    ac, as_ = np.ascontiguousarray(a.codes), np.ascontiguousarray(a.scales)
    bc, bs = np.ascontiguousarray(b.codes), np.ascontiguousarray(b.scales)
    rc = _load().orc_mx_gemm_entries(_ptr(ac, _u8p), _ptr(as_, _u8p), _ptr(bc, _u8p),
                                     _ptr(bs, _u8p), a.k, _ptr(ms, _i64p), _ptr(ns, _i64p),
                                     ms.size, _ptr(c, _f64p), _ptr(t, _f64p))
    if rc != 0:
        raise ValueError(f"oracle mx_gemm rejected the arguments (status {rc})")
    return c, t
