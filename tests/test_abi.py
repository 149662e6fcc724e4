"""The C-ABI library loads, exports every symbol include/nvfp4.h declares,
and rejects bad arguments before touching the GPU.  CPU only: every call
here fails validation, which returns before any HIP call."""
import ctypes
import os
import re

import pytest

import bit_microscaled_numerics_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nv.LIB_PATH):
        from bit_microscaled_numerics_amd import build
        build.build()
    return nv.load_library()


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+((?:nvfp4|mxfp4)_\w+)\s*\(", text,
                                 re.M)))


def test_header_and_binding_agree():
    assert declared() == sorted(nv.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in [(0, "NVFP4_OK"), (-1, "NVFP4_ERR_NULL"), (-2, "NVFP4_ERR_SHAPE"),
                       (-3, "NVFP4_ERR_ALIGN"), (-4, "NVFP4_ERR_ARG"), (-5, "NVFP4_ERR_LAUNCH")]:
        assert lib.nvfp4_status_string(code).decode() == name


FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MIS = 0x10001


def test_amax_validation(lib):
    assert lib.nvfp4_amax(None, 16, 16, FAKE, None) == nv.NVFP4_ERR_NULL
    assert lib.nvfp4_amax(FAKE, 16, 24, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_amax(FAKE, 0, 16, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_amax(FAKE, -16, 16, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_amax(FAKE, 16, (1 << 28) + 16, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_amax(MIS, 16, 16, FAKE, None) == nv.NVFP4_ERR_ALIGN
    assert lib.nvfp4_amax(FAKE, 16, 16, None, None) == nv.NVFP4_ERR_NULL
    assert "16" in lib.nvfp4_last_error().decode() or lib.nvfp4_last_error()


def test_quantize_validation(lib):
    q1 = lib.nvfp4_quantize1d_rtn
    assert q1(FAKE, 16, 16, 0, FAKE, 0, None, FAKE, FAKE, None) == nv.NVFP4_ERR_NULL
    assert q1(FAKE, 16, 16, 0, FAKE, 0, FAKE, None, FAKE, None) == nv.NVFP4_ERR_NULL
    assert q1(FAKE, 16, 16, 0, None, 0, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_NULL
    assert q1(FAKE, 16, 16, 0, FAKE, 0, FAKE, FAKE, None, None) == nv.NVFP4_ERR_NULL
    assert q1(FAKE, 16, 16, 0, FAKE, 0, MIS, FAKE, FAKE, None) == nv.NVFP4_ERR_ALIGN
    assert q1(FAKE, 16, 16, 2, FAKE, 0, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_ARG
    assert q1(FAKE, 16, 16, 0, FAKE, 2, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_ARG
    assert q1(FAKE, 17, 16, 0, FAKE, 0, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_SHAPE
    qs = lib.nvfp4_quantize1d_sr
    assert qs(FAKE, 16, 16, 5, FAKE, 0, 1, 0, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_ARG
    q2 = lib.nvfp4_quantize2d_rtn
    assert q2(FAKE, 16, 8, FAKE, 0, FAKE, None, FAKE, None, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert q2(FAKE, 16, 16, FAKE, 0, FAKE, MIS, FAKE, None, FAKE, None) == nv.NVFP4_ERR_ALIGN
    assert q2(FAKE, 16, 16, FAKE, 3, FAKE, None, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_ARG
    q2s = lib.nvfp4_quantize2d_sr
    assert q2s(None, 16, 16, FAKE, 0, 1, 0, FAKE, None, FAKE, None, FAKE, None) == nv.NVFP4_ERR_NULL
    r = lib.nvfp4_rht_quantize
    assert r(FAKE, 16, 16, 1, 2, 1, 0, FAKE, 0, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_ARG
    assert r(FAKE, 8, 16, 1, 0, 1, 0, FAKE, 0, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_amax_rht(FAKE, 16, 16, 1, None, None) == nv.NVFP4_ERR_NULL


def _op(**kw):
    base = dict(codes=FAKE, ld_codes=16, scales=FAKE, ss_row=2, ss_k=1, blk_rows=1,
                tensor_scale=FAKE, rows=16, k=32)
    base.update(kw)
    return nv.c_operand(**base)


def test_gemm_validation(lib):
    g = lib.nvfp4_gemm
    ok = _op()
    assert g(None, ctypes.byref(ok), FAKE, 16, None) == nv.NVFP4_ERR_NULL
    assert g(ctypes.byref(ok), ctypes.byref(_op(k=48)), FAKE, 16, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(_op(ld_codes=20)), FAKE, 16, None) == nv.NVFP4_ERR_ALIGN
    assert g(ctypes.byref(ok), ctypes.byref(_op(k=48, ld_codes=32)), FAKE, 16,
             None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(_op(rows=24)), FAKE, 24, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(_op(codes=MIS)), FAKE, 16, None) == nv.NVFP4_ERR_ALIGN
    assert g(ctypes.byref(ok), ctypes.byref(_op(blk_rows=4)), FAKE, 16, None) == nv.NVFP4_ERR_ARG
    assert g(ctypes.byref(ok), ctypes.byref(_op(scales=None)), FAKE, 16, None) == nv.NVFP4_ERR_NULL
    assert g(ctypes.byref(ok), ctypes.byref(ok), None, 16, None) == nv.NVFP4_ERR_NULL
    assert g(ctypes.byref(ok), ctypes.byref(ok), FAKE, 8, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(_op(ss_k=-1)), FAKE, 16, None) == nv.NVFP4_ERR_ARG
    assert lib.nvfp4_dequantize(ctypes.byref(ok), None, None) == nv.NVFP4_ERR_NULL
    assert lib.nvfp4_dequantize(ctypes.byref(ok), MIS, None) == nv.NVFP4_ERR_ALIGN


def test_python_layer_refuses_cpu_tensors():
    import torch
    x = torch.zeros(16, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv.quantize_1d(x)


def _mx(**kw):
    base = dict(codes=FAKE, ld_codes=32, scales=FAKE, ld_scales=2, rows=16, k=64)
    base.update(kw)
    return nv.c_mx_operand(**base)


def test_mxfp4_validation(lib):
    q = lib.mxfp4_quantize
    assert q(None, 16, 64, 0, 1, 0, FAKE, FAKE, None) == nv.NVFP4_ERR_NULL
    assert q(FAKE, 16, 48, 0, 1, 0, FAKE, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert q(FAKE, 0, 64, 0, 1, 0, FAKE, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert q(MIS, 16, 64, 0, 1, 0, FAKE, FAKE, None) == nv.NVFP4_ERR_ALIGN
    assert q(FAKE, 16, 64, 2, 1, 0, FAKE, FAKE, None) == nv.NVFP4_ERR_ARG
    g, d = lib.mxfp4_gemm, lib.mxfp4_dequantize
    ok = _mx()
    assert g(None, ctypes.byref(ok), FAKE, 16, None) == nv.NVFP4_ERR_NULL
    assert g(ctypes.byref(ok), ctypes.byref(_mx(k=96, ld_codes=48, ld_scales=3)), FAKE, 16,
             None) == nv.NVFP4_ERR_SHAPE                                   # a.k != b.k
    assert g(ctypes.byref(ok), ctypes.byref(_mx(k=48)), FAKE, 16, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(_mx(ld_codes=24)), FAKE, 16, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(_mx(ld_codes=40)), FAKE, 16, None) == nv.NVFP4_ERR_ALIGN
    assert g(ctypes.byref(ok), ctypes.byref(_mx(ld_scales=1)), FAKE, 16, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(ok), FAKE, 8, None) == nv.NVFP4_ERR_SHAPE   # ldc < N
    assert g(ctypes.byref(ok), ctypes.byref(ok), None, 16, None) == nv.NVFP4_ERR_NULL
    assert d(ctypes.byref(ok), MIS, None) == nv.NVFP4_ERR_ALIGN
    assert d(ctypes.byref(_mx(codes=None)), FAKE, None) == nv.NVFP4_ERR_NULL


def test_linear_rejects_cpu_tensors():
    """The training layer has no CPU path: CPU tensors are refused before any
    library call."""
    from bit_microscaled_numerics_amd import linear as L
    import torch
    x = torch.zeros(16, 32, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        L.linear_fwd_bwd(x, torch.zeros(16, 32, dtype=torch.bfloat16), x[:, :16].contiguous(), 1, 1)


def test_gemm_bf16_validation(lib):
    g = lib.nvfp4_gemm_bf16
    ok = _op()
    r = ctypes.byref
    assert g(r(ok), r(ok), None, 16, None, None, 0, None) == nv.NVFP4_ERR_NULL
    assert g(r(ok), r(ok), MIS, 16, None, None, 0, None) == nv.NVFP4_ERR_ALIGN
    assert g(r(ok), r(ok), FAKE, 16, MIS, None, 0, None) == nv.NVFP4_ERR_ALIGN
    assert g(r(ok), r(ok), FAKE, 8, None, None, 0, None) == nv.NVFP4_ERR_SHAPE
    assert g(r(ok), r(_op(k=48)), FAKE, 16, None, None, 0, None) == nv.NVFP4_ERR_SHAPE
    # a workspace size without a workspace; a workspace off 256-byte alignment
    assert g(r(ok), r(ok), FAKE, 16, None, None, 4096, None) == nv.NVFP4_ERR_ARG
    assert g(r(ok), r(ok), FAKE, 16, None, FAKE + 16, 4096, None) == nv.NVFP4_ERR_ALIGN


def test_gemm_bf16_noalloc_validation(lib):
    """The allocation-free variant: the same argument checks, its fixed
    workspace size, and the workspace query's refusal of empty shapes."""
    g = lib.nvfp4_gemm_bf16_noalloc
    ok = _op()
    r = ctypes.byref
    assert g(r(ok), r(ok), None, 16, None, None) == nv.NVFP4_ERR_NULL
    assert g(r(ok), r(ok), MIS, 16, None, None) == nv.NVFP4_ERR_ALIGN
    assert g(r(ok), r(ok), FAKE, 16, MIS, None) == nv.NVFP4_ERR_ALIGN
    assert g(r(ok), r(ok), FAKE, 8, None, None) == nv.NVFP4_ERR_SHAPE
    assert g(r(ok), r(_op(k=48)), FAKE, 16, None, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_gemm_bf16_noalloc_max_bytes() == 128 * 2 * 65536 * 4 + 128 * 4
    w = lib.nvfp4_gemm_bf16_workspace_bytes
    assert w(0, 16, 16) == nv.NVFP4_ERR_SHAPE
    assert w(16, -16, 16) == nv.NVFP4_ERR_SHAPE


def test_probe_mfma_validation(lib):
    """The measurement probe refuses bad arguments before touching the device."""
    p = lib.nvfp4_probe_mfma
    n = lib.nvfp4_probe_scratch_bytes()
    assert n > 0
    assert p(1, 100, None, n, None) == nv.NVFP4_ERR_NULL
    assert p(1, 100, FAKE + 16, n, None) == nv.NVFP4_ERR_ALIGN
    assert p(1, 100, FAKE, n - 1, None) == nv.NVFP4_ERR_SHAPE
    assert p(3, 100, FAKE, n, None) == nv.NVFP4_ERR_ARG
    assert p(-1, 100, FAKE, n, None) == nv.NVFP4_ERR_ARG
    assert p(1, 0, FAKE, n, None) == nv.NVFP4_ERR_ARG


def test_amax_both_validation(lib):
    f = lib.nvfp4_amax_both
    assert f(FAKE, 32, 16, 1, None, FAKE, None) == nv.NVFP4_ERR_NULL
    assert f(FAKE, 32, 16, 1, FAKE, None, None) == nv.NVFP4_ERR_NULL
    assert f(FAKE, 32, 16, 1, FAKE, FAKE, None) == nv.NVFP4_ERR_ARG
    assert f(FAKE, 32, 16, 1, MIS, FAKE + 16, None) == nv.NVFP4_ERR_ALIGN


def test_quantize_row_rht_validation(lib):
    f = lib.nvfp4_quantize_row_rht
    args = [FAKE, 32, 16, 1, 0, 0, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    a = list(args); a[10] = None   # codes_row
    assert f(*a) == nv.NVFP4_ERR_NULL
    a = list(args); a[13] = None   # codes_rht
    assert f(*a) == nv.NVFP4_ERR_NULL
    a = list(args); a[10] = MIS
    assert f(*a) == nv.NVFP4_ERR_ALIGN
    a = list(args); a[4] = 2       # use_sr
    assert f(*a) == nv.NVFP4_ERR_ARG
    a = list(args); a[1] = 24      # rows not a multiple of 16
    assert f(*a) == nv.NVFP4_ERR_SHAPE


def test_rht1d_validation(lib):
    """Both axes of the RHT entry points validate before launching; the
    COLWISE axis forwards to nvfp4_amax_rht / nvfp4_rht_quantize."""
    a = lib.nvfp4_amax_rht1d
    for axis in (0, 1):
        assert a(None, 16, 16, axis, 1, FAKE, None) == nv.NVFP4_ERR_NULL
        assert a(FAKE, 16, 24, axis, 1, FAKE, None) == nv.NVFP4_ERR_SHAPE
        assert a(MIS, 16, 16, axis, 1, FAKE, None) == nv.NVFP4_ERR_ALIGN
        assert a(FAKE, 16, 16, axis, 1, None, None) == nv.NVFP4_ERR_NULL
    assert a(FAKE, 16, 16, 2, 1, FAKE, None) == nv.NVFP4_ERR_ARG
    q = lib.nvfp4_rht_quantize1d
    args = [FAKE, 32, 16, 0, 1, 0, 0, 0, FAKE, 0, FAKE, FAKE, FAKE, None]
    for axis in (0, 1):
        b = list(args); b[3] = axis
        c = list(b); c[10] = None          # codes
        assert q(*c) == nv.NVFP4_ERR_NULL
        c = list(b); c[10] = MIS
        assert q(*c) == nv.NVFP4_ERR_ALIGN
        c = list(b); c[5] = 2              # use_sr
        assert q(*c) == nv.NVFP4_ERR_ARG
        c = list(b); c[9] = 2              # amax_mode
        assert q(*c) == nv.NVFP4_ERR_ARG
        c = list(b); c[2] = 8              # cols
        assert q(*c) == nv.NVFP4_ERR_SHAPE
        c = list(b); c[8] = None           # amax_io
        assert q(*c) == nv.NVFP4_ERR_NULL
    b = list(args); b[3] = -1
    assert q(*b) == nv.NVFP4_ERR_ARG


def test_measurement_probe_validation(lib):
    assert lib.nvfp4_probe_clock_bytes() >= 256 * 32
    c = lib.nvfp4_probe_clock
    assert c(None, 4096, None) == nv.NVFP4_ERR_NULL
    assert c(FAKE + 4, 4096, None) == nv.NVFP4_ERR_ALIGN
    assert c(FAKE, 16, None) == nv.NVFP4_ERR_SHAPE
    assert c(FAKE, 256 * 32 - 8, None) == nv.NVFP4_ERR_SHAPE
    p = lib.nvfp4_probe_copy
    assert p(None, FAKE, 16, None) == nv.NVFP4_ERR_NULL
    assert p(FAKE, MIS, 16, None) == nv.NVFP4_ERR_ALIGN
    assert p(FAKE, FAKE + 4096, 24, None) == nv.NVFP4_ERR_SHAPE
    assert p(FAKE, FAKE + 4096, 0, None) == nv.NVFP4_ERR_SHAPE
    assert p(FAKE, FAKE + 4096, (1 << 40) + 16, None) == nv.NVFP4_ERR_SHAPE


def test_sizes_beyond_2_pow_40_are_rejected(lib):
    """Dimensions that are multiples of 16 but whose products overflow the
    library's size bound are rejected before any arithmetic on them."""
    big = 1 << 62
    assert lib.nvfp4_amax(FAKE, big, 1 << 28, FAKE, None) == nv.NVFP4_ERR_SHAPE
    assert lib.nvfp4_quantize1d_rtn(FAKE, big, 1 << 20, 0, FAKE, 0, FAKE, FAKE, FAKE,
                                    None) == nv.NVFP4_ERR_SHAPE
    g = lib.nvfp4_gemm
    ok = _op()
    assert g(ctypes.byref(_op(rows=big)), ctypes.byref(ok), FAKE, 16, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(_op(ss_row=big)), ctypes.byref(ok), FAKE, 16, None) == nv.NVFP4_ERR_SHAPE
    assert g(ctypes.byref(ok), ctypes.byref(ok), FAKE, big, None) == nv.NVFP4_ERR_SHAPE
