"""NVFP4 quantization and the NVFP4-linear GEMM on MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so`` (C ABI in ``include/nvfp4.h``).
PyTorch provides device memory and the current HIP stream; every step of the
path runs in the library's HIP kernels.  There is no CPU fallback: if the
library is missing or no GPU is present, calls raise.

Two layers:
  * ``nvfp4_*`` functions with the C names and arguments (torch tensors in
    place of pointers), for callers that manage their own buffers;
  * ``quantize_1d`` / ``quantize_2d`` / ``rht_quantize`` / ``dequantize`` /
    ``gemm``, which allocate outputs with ``torch.empty`` and return
    :class:`NVFP4Tensor` operands.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK, NVFP4_ERR_NULL, NVFP4_ERR_SHAPE, NVFP4_ERR_ALIGN, NVFP4_ERR_ARG, NVFP4_ERR_LAUNCH = (
    0, -1, -2, -3, -4, -5)
NVFP4_AMAX_COMPUTE, NVFP4_AMAX_GIVEN = 0, 1
NVFP4_ROWWISE, NVFP4_COLWISE = 0, 1

EXPORTED = ("nvfp4_amax", "nvfp4_amax_rht", "nvfp4_quantize1d_rtn", "nvfp4_quantize1d_sr",
            "nvfp4_quantize2d_rtn", "nvfp4_quantize2d_sr", "nvfp4_rht_quantize",
            "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_status_string", "nvfp4_last_error",
            "nvfp4_gemm_bf16", "nvfp4_gemm_bf16_workspace_bytes", "nvfp4_gemm_bf16_noalloc",
            "nvfp4_gemm_bf16_noalloc_max_bytes", "mxfp4_quantize", "mxfp4_dequantize", "mxfp4_gemm",
            "nvfp4_probe_mfma", "nvfp4_probe_scratch_bytes", "nvfp4_amax_both",
            "nvfp4_quantize_row_rht", "nvfp4_amax_rht1d", "nvfp4_rht_quantize1d",
            "nvfp4_probe_clock", "nvfp4_probe_clock_bytes", "nvfp4_probe_copy")


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} ({status})")
        self.status = status


class c_operand(ctypes.Structure):
    """Mirror of ``nvfp4_operand``."""
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ss_row", ctypes.c_int64),
                ("ss_k", ctypes.c_int64), ("blk_rows", ctypes.c_int32),
                ("tensor_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("k", ctypes.c_int64)]


class c_mx_operand(ctypes.Structure):
    """Mirror of ``mxfp4_operand``."""
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ld_scales", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("k", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnvfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           f"`python -m bit_microscaled_numerics_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, u64, u32, i32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                              ctypes.c_uint32, ctypes.c_int)
    sigs = {
        "nvfp4_amax": [vp, i64, i64, vp, vp],
        "nvfp4_amax_rht": [vp, i64, i64, u64, vp, vp],
        "nvfp4_amax_both": [vp, i64, i64, u64, vp, vp, vp],
        "nvfp4_quantize1d_rtn": [vp, i64, i64, i32, vp, i32, vp, vp, vp, vp],
        "nvfp4_quantize1d_sr": [vp, i64, i64, i32, vp, i32, u64, u32, vp, vp, vp, vp],
        "nvfp4_quantize2d_rtn": [vp, i64, i64, vp, i32, vp, vp, vp, vp, vp, vp],
        "nvfp4_quantize2d_sr": [vp, i64, i64, vp, i32, u64, u32, vp, vp, vp, vp, vp, vp],
        "nvfp4_rht_quantize": [vp, i64, i64, u64, i32, u64, u32, vp, i32, vp, vp, vp, vp],
        "nvfp4_amax_rht1d": [vp, i64, i64, i32, u64, vp, vp],
        "nvfp4_rht_quantize1d": [vp, i64, i64, i32, u64, i32, u64, u32, vp, i32, vp, vp, vp, vp],
        "nvfp4_quantize_row_rht": [vp, i64, i64, u64, i32, u64, u32, u32, vp, vp, vp, vp, vp, vp,
                                   vp, vp, vp],
        "nvfp4_dequantize": [ctypes.POINTER(c_operand), vp, vp],
        "nvfp4_gemm": [ctypes.POINTER(c_operand), ctypes.POINTER(c_operand), vp, i64, vp],
        "nvfp4_gemm_bf16": [ctypes.POINTER(c_operand), ctypes.POINTER(c_operand), vp, i64, vp, vp,
                            i64, vp],
        "nvfp4_gemm_bf16_noalloc": [ctypes.POINTER(c_operand), ctypes.POINTER(c_operand), vp, i64,
                                    vp, vp],
        "mxfp4_quantize": [vp, i64, i64, i32, u64, u32, vp, vp, vp],
        "mxfp4_dequantize": [ctypes.POINTER(c_mx_operand), vp, vp],
        "mxfp4_gemm": [ctypes.POINTER(c_mx_operand), ctypes.POINTER(c_mx_operand), vp, i64, vp],
        "nvfp4_probe_mfma": [i32, i32, vp, i64, vp],
        "nvfp4_probe_clock": [vp, i64, vp],
        "nvfp4_probe_copy": [vp, vp, i64, vp],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.nvfp4_status_string.argtypes = [ctypes.c_int]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_last_error.argtypes = []
    lib.nvfp4_last_error.restype = ctypes.c_char_p
    for name in ("nvfp4_probe_scratch_bytes", "nvfp4_probe_clock_bytes",
                 "nvfp4_gemm_bf16_noalloc_max_bytes"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = ctypes.c_int64
    lib.nvfp4_gemm_bf16_workspace_bytes.argtypes = [i64, i64, i64]
    lib.nvfp4_gemm_bf16_workspace_bytes.restype = ctypes.c_int64
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != NVFP4_OK:
        lib = load_library()
        raise NVFP4Error(status, f"{lib.nvfp4_status_string(status).decode()}: "
                                 f"{lib.nvfp4_last_error().decode()}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _empty(*shape, dtype, device) -> torch.Tensor:
    """Every output buffer of the allocating functions below comes from here
    (one place to replace the allocator, e.g. with guard-banded buffers)."""
    return torch.empty(*shape, dtype=dtype, device=device)


def _dev_bf16(x: torch.Tensor, name: str):
    if not x.is_cuda or x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D bf16 CUDA tensor")


# --------------------------------------------------------------------------- C names
def nvfp4_amax(x, amax_out, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_amax(_p(x), x.shape[0], x.shape[1], _p(amax_out), _stream(stream)))


def nvfp4_amax_both(x, rht_seed, amax_out, amax_rht_out, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_amax_both(_p(x), x.shape[0], x.shape[1], rht_seed, _p(amax_out),
                                          _p(amax_rht_out), _stream(stream)))


def nvfp4_amax_rht(x, rht_seed, amax_out, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_amax_rht(_p(x), x.shape[0], x.shape[1], rht_seed, _p(amax_out),
                                         _stream(stream)))


def nvfp4_quantize1d_rtn(x, axis, amax_io, amax_mode, codes, scales, ts_out, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_quantize1d_rtn(_p(x), x.shape[0], x.shape[1], axis, _p(amax_io),
                                               amax_mode, _p(codes), _p(scales), _p(ts_out),
                                               _stream(stream)))


def nvfp4_quantize1d_sr(x, axis, amax_io, amax_mode, seed, stream_id, codes, scales, ts_out,
                        stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_quantize1d_sr(_p(x), x.shape[0], x.shape[1], axis, _p(amax_io),
                                              amax_mode, seed, stream_id, _p(codes), _p(scales),
                                              _p(ts_out), _stream(stream)))


def nvfp4_quantize2d_rtn(w, amax_io, amax_mode, codes, codes_t, scales, scales_t, ts_out,
                         stream=None):
    _dev_bf16(w, "w")
    _check(load_library().nvfp4_quantize2d_rtn(_p(w), w.shape[0], w.shape[1], _p(amax_io),
                                               amax_mode, _p(codes), _p(codes_t), _p(scales),
                                               _p(scales_t), _p(ts_out), _stream(stream)))


def nvfp4_quantize2d_sr(w, amax_io, amax_mode, seed, stream_id, codes, codes_t, scales, scales_t,
                        ts_out, stream=None):
    _dev_bf16(w, "w")
    _check(load_library().nvfp4_quantize2d_sr(_p(w), w.shape[0], w.shape[1], _p(amax_io),
                                              amax_mode, seed, stream_id, _p(codes), _p(codes_t),
                                              _p(scales), _p(scales_t), _p(ts_out),
                                              _stream(stream)))


def nvfp4_rht_quantize(x, rht_seed, use_sr, sr_seed, stream_id, amax_io, amax_mode, codes,
                       scales, ts_out, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_rht_quantize(_p(x), x.shape[0], x.shape[1], rht_seed,
                                             int(use_sr), sr_seed, stream_id, _p(amax_io),
                                             amax_mode, _p(codes), _p(scales), _p(ts_out),
                                             _stream(stream)))


def nvfp4_amax_rht1d(x, axis, rht_seed, amax_out, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_amax_rht1d(_p(x), x.shape[0], x.shape[1], axis, rht_seed,
                                           _p(amax_out), _stream(stream)))


def nvfp4_rht_quantize1d(x, axis, rht_seed, use_sr, sr_seed, stream_id, amax_io, amax_mode, codes,
                         scales, ts_out, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_rht_quantize1d(_p(x), x.shape[0], x.shape[1], axis, rht_seed,
                                               int(use_sr), sr_seed, stream_id, _p(amax_io),
                                               amax_mode, _p(codes), _p(scales), _p(ts_out),
                                               _stream(stream)))


def nvfp4_quantize_row_rht(x, rht_seed, use_sr, sr_seed, stream_id_row, stream_id_rht, amax_row,
                           amax_rht, codes_row, scales_row, ts_row, codes_rht, scales_rht, ts_rht,
                           stream=None):
    _dev_bf16(x, "x")
    _check(load_library().nvfp4_quantize_row_rht(
        _p(x), x.shape[0], x.shape[1], rht_seed, int(use_sr), sr_seed, stream_id_row,
        stream_id_rht, _p(amax_row), _p(amax_rht), _p(codes_row), _p(scales_row), _p(ts_row),
        _p(codes_rht), _p(scales_rht), _p(ts_rht), _stream(stream)))


def nvfp4_dequantize(q: "NVFP4Tensor", out, stream=None):
    op = q.c_struct()
    _check(load_library().nvfp4_dequantize(ctypes.byref(op), _p(out), _stream(stream)))


def nvfp4_gemm(a: "NVFP4Tensor", b: "NVFP4Tensor", c, ldc: int, stream=None):
    oa, ob = a.c_struct(), b.c_struct()
    _check(load_library().nvfp4_gemm(ctypes.byref(oa), ctypes.byref(ob), _p(c), ldc,
                                     _stream(stream)))


# --------------------------------------------------------------------------- operands
@dataclass
class NVFP4Tensor:
    """A quantized operand, logically [rows][k], K-contiguous (device tensors)."""
    codes: torch.Tensor          # uint8 [rows][ld_codes]
    scales: torch.Tensor         # uint8 E4M3 codes
    tensor_scale: torch.Tensor   # float32 [1]
    amax: torch.Tensor           # float32 [1]
    rows: int
    k: int
    blk_rows: int = 1
    ss_row: int = 0
    ss_k: int = 1
    codes_t: Optional[torch.Tensor] = None   # 2D weights: the same codes transposed
    scales_t: Optional[torch.Tensor] = None  # 2D weights: the scale matrix transposed

    def c_struct(self) -> c_operand:
        return c_operand(self.codes.data_ptr(), self.codes.shape[1], self.scales.data_ptr(),
                         self.ss_row, self.ss_k, self.blk_rows, self.tensor_scale.data_ptr(),
                         self.rows, self.k)

    def t(self) -> "NVFP4Tensor":
        """A 2D-quantized weight read as its transpose (the Dgrad operand)."""
        if self.blk_rows != 16 or self.codes_t is None:
            raise ValueError("only 2D operands quantized with codes_t can be transposed")
        if self.scales_t is not None:  # K-contiguous scales (the GEMM's fast path)
            return NVFP4Tensor(self.codes_t, self.scales_t, self.tensor_scale, self.amax, self.k,
                               self.rows, 16, self.rows // 16, 1, self.codes, self.scales)
        return NVFP4Tensor(self.codes_t, self.scales, self.tensor_scale, self.amax, self.k,
                           self.rows, 16, self.ss_k, self.ss_row, self.codes)

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel()


def _outputs(I, K, dev, scale_shape):
    codes = _empty(I, K // 2, dtype=torch.uint8, device=dev)
    scales = _empty(*scale_shape, dtype=torch.uint8, device=dev)
    ts = _empty(1, dtype=torch.float32, device=dev)
    return codes, scales, ts


def _amax_arg(x, amax):
    if amax is None:
        return _empty(1, dtype=torch.float32, device=x.device), NVFP4_AMAX_COMPUTE
    if isinstance(amax, torch.Tensor):
        return amax, NVFP4_AMAX_GIVEN
    return torch.tensor([float(amax)], dtype=torch.float32, device=x.device), NVFP4_AMAX_GIVEN


def amax(x: torch.Tensor) -> torch.Tensor:
    out = _empty(1, dtype=torch.float32, device=x.device)
    nvfp4_amax(x, out)
    return out


def amax_rht(x: torch.Tensor, rht_seed: int, axis: int = NVFP4_COLWISE) -> torch.Tensor:
    """max |RHT(x)| with the transform along the rows (COLWISE, the Wgrad
    layout) or along each row (ROWWISE)."""
    out = _empty(1, dtype=torch.float32, device=x.device)
    nvfp4_amax_rht1d(x, axis, rht_seed, out)
    return out


def amax_both(x: torch.Tensor, rht_seed: int):
    """(max |x|, max |RHT(x^T)|) from one read of x, as two 1-element tensors."""
    out = _empty(2, dtype=torch.float32, device=x.device)
    nvfp4_amax_both(x, rht_seed, out[0:1], out[1:2])
    return out[0:1], out[1:2]


def quantize_1d(x: torch.Tensor, axis: int = NVFP4_ROWWISE, sr_seed: Optional[int] = None,
                stream_id: int = 0, amax=None) -> NVFP4Tensor:
    """1D (16 along K) quantization; COLWISE gives the quantized transpose."""
    _dev_bf16(x, "x")
    R, C = x.shape
    I, K = (C, R) if axis == NVFP4_COLWISE else (R, C)
    codes, scales, ts = _outputs(I, K, x.device, (I, K // 16))
    am, mode = _amax_arg(x, amax)
    if sr_seed is None:
        nvfp4_quantize1d_rtn(x, axis, am, mode, codes, scales, ts)
    else:
        nvfp4_quantize1d_sr(x, axis, am, mode, sr_seed, stream_id, codes, scales, ts)
    return NVFP4Tensor(codes, scales, ts, am, I, K, 1, K // 16, 1)


def quantize_2d(w: torch.Tensor, sr_seed: Optional[int] = None, stream_id: int = 0,
                with_codes_t: bool = True, amax=None) -> NVFP4Tensor:
    """2D (16x16 tile) quantization of a weight [rows][cols]."""
    _dev_bf16(w, "w")
    R, C = w.shape
    codes, scales, ts = _outputs(R, C, w.device, (R // 16, C // 16))
    codes_t = scales_t = None
    if with_codes_t:
        codes_t = _empty(C, R // 2, dtype=torch.uint8, device=w.device)
        scales_t = _empty(C // 16, R // 16, dtype=torch.uint8, device=w.device)
    am, mode = _amax_arg(w, amax)
    if sr_seed is None:
        nvfp4_quantize2d_rtn(w, am, mode, codes, codes_t, scales, scales_t, ts)
    else:
        nvfp4_quantize2d_sr(w, am, mode, sr_seed, stream_id, codes, codes_t, scales, scales_t, ts)
    return NVFP4Tensor(codes, scales, ts, am, R, C, 16, C // 16, 1, codes_t, scales_t)


def rht_quantize(x: torch.Tensor, rht_seed: int, sr_seed: Optional[int] = None,
                 stream_id: int = 0, amax=None, axis: int = NVFP4_COLWISE) -> NVFP4Tensor:
    """1D quantization of the 16-point RHT of x.  COLWISE (the Wgrad operand):
    the quantized transpose, transform along the rows (tokens).  ROWWISE
    (Fprop / Dgrad operands with the transform along K): transform along
    each row, codes [rows][cols/2]."""
    _dev_bf16(x, "x")
    R, C = x.shape
    I, K = (C, R) if axis == NVFP4_COLWISE else (R, C)
    codes, scales, ts = _outputs(I, K, x.device, (I, K // 16))
    am, mode = _amax_arg(x, amax)
    nvfp4_rht_quantize1d(x, axis, rht_seed, sr_seed is not None,
                         0 if sr_seed is None else sr_seed, stream_id, am, mode, codes, scales, ts)
    return NVFP4Tensor(codes, scales, ts, am, I, K, 1, K // 16, 1)


def quantize_row_rht(x: torch.Tensor, rht_seed: int, sr_seed: Optional[int] = None,
                     stream_ids=(0, 1)):
    """(rowwise 1D operand of x, Wgrad operand RHT(x)^T) from one read of x,
    byte-identical to quantize_1d(x, ...) and rht_quantize(x, ...) with the
    same seeds and stream ids; the two amaxes come from one amax_both pass."""
    _dev_bf16(x, "x")
    R, C = x.shape
    am_row, am_rht = amax_both(x, rht_seed)
    codes_r, scales_r, ts_r = _outputs(R, C, x.device, (R, C // 16))
    codes_t, scales_t, ts_t = _outputs(C, R, x.device, (C, R // 16))
    nvfp4_quantize_row_rht(x, rht_seed, sr_seed is not None, 0 if sr_seed is None else sr_seed,
                           stream_ids[0], stream_ids[1], am_row, am_rht, codes_r, scales_r, ts_r,
                           codes_t, scales_t, ts_t)
    return (NVFP4Tensor(codes_r, scales_r, ts_r, am_row, R, C, 1, C // 16, 1),
            NVFP4Tensor(codes_t, scales_t, ts_t, am_rht, C, R, 1, R // 16, 1))


def dequantize(q: NVFP4Tensor) -> torch.Tensor:
    out = _empty(q.rows, q.k, dtype=torch.float32, device=q.codes.device)
    nvfp4_dequantize(q, out)
    return out


def nvfp4_gemm_bf16(a: "NVFP4Tensor", b: "NVFP4Tensor", c, ldc: int, amax_out=None,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    oa, ob = a.c_struct(), b.c_struct()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().nvfp4_gemm_bf16(ctypes.byref(oa), ctypes.byref(ob), _p(c), ldc,
                                          _p(amax_out), _p(workspace), nbytes, _stream(stream)))


def nvfp4_gemm_bf16_workspace_bytes(M: int, N: int, K: int) -> int:
    n = int(load_library().nvfp4_gemm_bf16_workspace_bytes(M, N, K))
    if n < 0:
        _check(n)
    return n


def nvfp4_gemm_bf16_noalloc(a: "NVFP4Tensor", b: "NVFP4Tensor", c, ldc: int, amax_out=None,
                            stream=None):
    oa, ob = a.c_struct(), b.c_struct()
    _check(load_library().nvfp4_gemm_bf16_noalloc(ctypes.byref(oa), ctypes.byref(ob), _p(c), ldc,
                                                  _p(amax_out), _stream(stream)))


def gemm_bf16_workspace(M: int, N: int, K: int, device) -> Optional[torch.Tensor]:
    """The workspace nvfp4_gemm_bf16 takes for an M x N x K product (None when
    it needs none); reusable by any later call of the same or smaller need on
    the same stream."""
    n = nvfp4_gemm_bf16_workspace_bytes(M, N, K)
    if n == 0:
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


def gemm_bf16(a: NVFP4Tensor, b: NVFP4Tensor, out: Optional[torch.Tensor] = None,
              with_amax: bool = True, workspace: Union[torch.Tensor, None, bool] = True):
    """C = s_a s_b A B^T rounded to BF16, and (with_amax) max |C| as a device
    float, ready to pass as the given amax of C's quantization.  workspace:
    True allocates the K-split workspace (every entry then equals the FP32
    GEMM's, rounded), a tensor supplies it, None/False runs without one."""
    if out is None:
        out = _empty(a.rows, b.rows, dtype=torch.bfloat16, device=a.codes.device)
    amax = _empty(1, dtype=torch.float32, device=a.codes.device) if with_amax else None
    if workspace is True:
        workspace = gemm_bf16_workspace(a.rows, b.rows, a.k, a.codes.device)
    elif workspace is False:
        workspace = None
    nvfp4_gemm_bf16(a, b, out, out.stride(0), amax, workspace)
    return out, amax


def gemm(a: NVFP4Tensor, b: NVFP4Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = s_a s_b A B^T in FP32, A [M][K], B [N][K]."""
    if out is None:
        out = _empty(a.rows, b.rows, dtype=torch.float32, device=a.codes.device)
    nvfp4_gemm(a, b, out, out.stride(0))
    return out


# ---------------------------------------------------------------- MXFP4
@dataclass
class MXFP4Tensor:
    """An MXFP4 operand, logically [rows][k], K-contiguous (device tensors)."""
    codes: torch.Tensor    # uint8 [rows][ld_codes]
    scales: torch.Tensor   # uint8 E8M0 [rows][ld_scales]
    rows: int
    k: int

    def c_struct(self) -> c_mx_operand:
        return c_mx_operand(self.codes.data_ptr(), self.codes.shape[1], self.scales.data_ptr(),
                            self.scales.shape[1], self.rows, self.k)


def mxfp4_quantize(x, use_sr, seed, stream_id, codes, scales, stream=None):
    _dev_bf16(x, "x")
    _check(load_library().mxfp4_quantize(_p(x), x.shape[0], x.shape[1], int(use_sr), seed,
                                         stream_id, _p(codes), _p(scales), _stream(stream)))


def mxfp4_dequantize(q: MXFP4Tensor, out, stream=None):
    op = q.c_struct()
    _check(load_library().mxfp4_dequantize(ctypes.byref(op), _p(out), _stream(stream)))


def mxfp4_gemm(a: MXFP4Tensor, b: MXFP4Tensor, c, ldc: int, stream=None):
    oa, ob = a.c_struct(), b.c_struct()
    _check(load_library().mxfp4_gemm(ctypes.byref(oa), ctypes.byref(ob), _p(c), ldc,
                                      _stream(stream)))


def mx_quantize(x: torch.Tensor, sr_seed: Optional[int] = None, stream_id: int = 0) -> MXFP4Tensor:
    """Rowwise MXFP4 quantization of bf16 x [rows][cols] (cols % 32 == 0)."""
    _dev_bf16(x, "x")
    R, C = x.shape
    codes = _empty(R, C // 2, dtype=torch.uint8, device=x.device)
    scales = _empty(R, C // 32, dtype=torch.uint8, device=x.device)
    mxfp4_quantize(x, sr_seed is not None, 0 if sr_seed is None else sr_seed, stream_id, codes,
                   scales)
    return MXFP4Tensor(codes, scales, R, C)


def mx_dequantize(q: MXFP4Tensor) -> torch.Tensor:
    out = _empty(q.rows, q.k, dtype=torch.float32, device=q.codes.device)
    mxfp4_dequantize(q, out)
    return out


def mx_gemm(a: MXFP4Tensor, b: MXFP4Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A B^T in FP32, A [M][K], B [N][K] MXFP4."""
    if out is None:
        out = _empty(a.rows, b.rows, dtype=torch.float32, device=a.codes.device)
    mxfp4_gemm(a, b, out, out.stride(0))
    return out


PROBE_ZEROS, PROBE_NVFP4_LIKE, PROBE_UNIFORM = 0, 1, 2


def probe_mfma(mode: int, iters: int = 8000):
    """(TFLOP/s, clock GHz) of the FP16 matrix cores running the GEMM's MFMA
    pattern from registers on operand data of kind ``mode`` (measurement
    support: the ceiling the GEMM's roofline fraction is read against).
    Synchronizes the device; the library call itself only enqueues."""
    lib = load_library()
    nbytes = int(lib.nvfp4_probe_scratch_bytes())
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    _check(lib.nvfp4_probe_mfma(mode, iters, _p(scratch), nbytes, _stream(None)))
    torch.cuda.synchronize()
    wgs = 256
    st = scratch[nbytes - wgs * 32:].view(torch.int64).cpu().view(wgs, 4).tolist()
    ghz = sum((t1 - t0) / (r1 - r0) * 0.1 for t0, t1, r0, r1 in st) / wgs
    secs = (max(r[3] for r in st) - min(r[2] for r in st)) * 1e-8
    flops = 2.0 * 32 * 32 * 16 * 16 * iters * 4 * wgs
    return flops / secs / 1e12, ghz


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Plain device copy of src's bytes into dst (measurement support)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _check(load_library().nvfp4_probe_copy(_p(src), _p(dst), n, _stream(stream)))


class ClockStamps:
    """Average shader clock of work enqueued between ``before()`` and
    ``after()`` on the current stream (measurement support): per compute
    unit, the difference of its shader-clock counter over that of the
    100 MHz real-time counter; the median over the CUs stamped both times.
    ``ghz()`` synchronizes."""

    def __init__(self, device="cuda"):
        lib = load_library()
        n = int(lib.nvfp4_probe_clock_bytes())
        self._n = n
        self._buf = torch.empty(2, n // 8, dtype=torch.int64, device=device)

    def _stamp(self, i: int, stream=None):
        _check(load_library().nvfp4_probe_clock(self._buf[i].data_ptr(), self._n, _stream(stream)))

    def before(self, stream=None):
        self._stamp(0, stream)

    def after(self, stream=None):
        self._stamp(1, stream)

    def ghz(self) -> float:
        torch.cuda.synchronize()
        st = self._buf.cpu().view(2, -1, 4).tolist()
        first, last = {}, {}
        for xcc, hw, t, r in st[0]:
            first.setdefault((xcc, hw & 0xFF00), (t, r))
        for xcc, hw, t, r in st[1]:
            last[(xcc, hw & 0xFF00)] = (t, r)
        rates = sorted((last[k][0] - first[k][0]) / (last[k][1] - first[k][1]) * 0.1
                       for k in first if k in last and last[k][1] > first[k][1])
        return rates[len(rates) // 2] if rates else float("nan")
