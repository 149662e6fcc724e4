#!/usr/bin/env python3
"""Benchmark: one NVFP4 linear-layer training step (Fprop, Dgrad, Wgrad with
all their quantizations) at the 12B hybrid's FFN down-projection shape,
8192 tokens x 20480 (FFN) -> 5120 (hidden), on one MI355X.

A step is the whole hot path over one batch of seeded synthetic inputs that
are resident in HBM before timing starts:
  Q(X)   rowwise 1D RTN and Q(RHT(X)^T) RTN: both amaxes in one read, both encodes in one read
  Q(W)   2D 16x16 RTN + transposed codes and scales (amax + encode)
  Fprop  Y  = Q(X) Q(W)^T        M=8192  N=5120  K=20480
  Q(dY)  rowwise 1D SR (both amaxes of dY in one read + encode)
  Dgrad  dX = Q(dY) Q(W)         M=8192  N=20480 K=5120
  Q(RHT(dY)^T) SR (encode)
  Wgrad  dW = dY^T X             M=5120  N=20480 K=8192
Outputs are preallocated; nothing is allocated inside the timed region.

Prints ONE JSON line.  `value` is whole-step NVFP4-linear throughput
(3 * 2MNK GEMM FLOP per step / step time, quantization included); per-kernel
GB/s and TFLOP/s (HIP events on the launch stream) are reported beside it, with
the roofline of the dominant kernel and the CPU oracle's rate on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bit_microscaled_numerics_amd as nv  # noqa: E402
from bit_microscaled_numerics_amd import inputs  # noqa: E402

METRIC = "NVFP4 quantize GB/s + NVFP4-linear GEMM TFLOP/s at 8192×5120×20480"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16/BF16 matrix peak
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 (scaled MX) matrix peak

TOKENS, HIDDEN, FFN = 8192, 5120, 20480
RHT_SEED, SR_SEED = 1, 1


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


GEMM_SOURCES = ("nvfp4_gemm.hip", "gemm_tiles.h", "gemm_decode.h", "nvfp4_device.h")
QUANT_SOURCES = ("nvfp4_quant.hip", "mxfp4.hip", "nvfp4_device.h", "gemm_tiles.h")
# VALU issue peak in lane-instructions per second: 1024 SIMDs, a wave64
# instruction every 4 cycles per SIMD (16 lanes a cycle), 2.4 GHz
VALU_LANE_OPS_PER_S = 1024 * 64 / 4 * 2.4e9


def gemm_source_digest() -> str:
    """SHA-256 of the GEMM sources with comments and blank lines removed, so
    that the record below goes stale when the code changes, not its comments."""
    return source_digest(GEMM_SOURCES)


def source_digest(files) -> str:
    import hashlib
    import re
    m = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_microscaled_numerics_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
        m.update("\n".join(ln for ln in lines if ln).encode())
    return m.hexdigest()


def gemm_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record, or None when the GEMM code changed since."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    return rec["traffic_bytes_per_launch"] if gemm_source_digest() == rec["source_sha256"] else None


# the sweep's stochastic-rounding encodes and the kernel each one launches
SR_SWEEP_KERNELS = {"1d SR encode": "k_quant_row<true, false>",
                    "row RHT SR encode": "k_quant_row<true, true>",
                    "col RHT SR encode": "k_quant_col<true, true, false>",
                    "MXFP4 SR (single pass)": "k_mx_quant_row<true>"}


def quant_valu():
    """VALU lane-instructions per 8 elements of the quantizer kernels, from the
    committed rocprofv3 SQ_INSTS_VALU record, or None when the quantizer code
    changed since."""
    path = os.path.join(ROOT, "profiles", "quantize_valu.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    return rec["valu_per_8_elements"] if source_digest(QUANT_SOURCES) == rec["source_sha256"] else None


class Flush:
    """Evicts the 256 MB Infinity Cache (and the L2s) between timed launches:
    a 1 GiB fill, outside the timed interval, so a kernel that re-reads a
    tensor another kernel has just read (an encode after its amax) is timed
    from HBM, not from the cache."""

    def __init__(self, nbytes: int = 1 << 30):
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.k = 0

    def __call__(self):
        self.k ^= 1
        self.buf.fill_(self.k)


def copy_peak(reps: int = 10):
    """HBM bandwidth of a plain device copy of 1 GiB (the library's probe
    copy kernel, the read pattern of the amax and rowwise kernels; torch's
    copy_ beside it): 2 GiB moved per launch; medians of `reps`."""
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    nbytes = 2.0 * src.numel() * 2
    ms = _median_ms(lambda: nv.probe_copy(src, dst), reps)
    ms_torch = _median_ms(lambda: dst.copy_(src), reps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 3), "bytes": int(nbytes),
            "kernel": "nvfp4_probe_copy of 1 GiB (read + write)",
            "torch_copy_GB/s": round(nbytes / (ms_torch * 1e-3) / 1e9, 1)}


class Step:
    """Preallocated buffers and the ordered list of launches of one step."""

    def __init__(self, x, w, dy):
        dev = x.device
        T, F = x.shape          # tokens, in-features (FFN)
        H = w.shape[0]          # out-features (hidden)
        self.x, self.w, self.dy = x, w, dy
        e = lambda *s, dt=torch.uint8: torch.empty(*s, dtype=dt, device=dev)  # noqa: E731
        f1 = lambda: torch.empty(1, dtype=torch.float32, device=dev)  # noqa: E731
        self.qx = nv.NVFP4Tensor(e(T, F // 2), e(T, F // 16), f1(), f1(), T, F, 1, F // 16, 1)
        self.qw = nv.NVFP4Tensor(e(H, F // 2), e(H // 16, F // 16), f1(), f1(), H, F, 16,
                                 F // 16, 1, e(F, H // 2), e(F // 16, H // 16))
        self.qdy = nv.NVFP4Tensor(e(T, H // 2), e(T, H // 16), f1(), f1(), T, H, 1, H // 16, 1)
        self.qdy_t = nv.NVFP4Tensor(e(H, T // 2), e(H, T // 16), f1(), f1(), H, T, 1, T // 16, 1)
        self.qx_t = nv.NVFP4Tensor(e(F, T // 2), e(F, T // 16), f1(), f1(), F, T, 1, T // 16, 1)
        self.y = e(T, H, dt=torch.float32)
        self.dx = e(T, F, dt=torch.float32)
        self.dw = e(H, F, dt=torch.float32)
        C, G = nv.NVFP4_AMAX_COMPUTE, nv.NVFP4_AMAX_GIVEN
        q = self
        n_x, n_w, n_dy = x.numel(), w.numel(), dy.numel()
        # (name, kind, algorithmic bytes or flops, callable); each launch is
        # timed on its own.  X and dY are quantized both plainly and under the
        # RHT, so one read gives both of their amaxes.
        self.ops = [
            ("amax X + RHT X", "hbm", 2 * n_x,
             lambda: nv.nvfp4_amax_both(x, RHT_SEED, q.qx.amax, q.qx_t.amax)),
            ("quant X rowwise + X^T RHT RTN", "hbm", 3.125 * n_x,
             lambda: nv.nvfp4_quantize_row_rht(x, RHT_SEED, 0, 0, 0, 0, q.qx.amax, q.qx_t.amax,
                                               q.qx.codes, q.qx.scales, q.qx.tensor_scale,
                                               q.qx_t.codes, q.qx_t.scales, q.qx_t.tensor_scale)),
            ("amax W", "hbm", 2 * n_w, lambda: nv.nvfp4_amax(w, q.qw.amax)),
            ("quant W 2D RTN +transposed", "hbm", 3.0078125 * n_w,
             lambda: nv.nvfp4_quantize2d_rtn(w, q.qw.amax, G, q.qw.codes, q.qw.codes_t,
                                             q.qw.scales, q.qw.scales_t, q.qw.tensor_scale)),
            ("gemm Fprop", "mfma", 2.0 * T * H * F, lambda: nv.gemm(q.qx, q.qw, q.y)),
            ("amax dY + RHT dY", "hbm", 2 * n_dy,
             lambda: nv.nvfp4_amax_both(dy, RHT_SEED, q.qdy.amax, q.qdy_t.amax)),
            # dY's two SR encodes stay separate launches: one shared pass
            # (nvfp4_quantize_row_rht with SR) saves only ~5 us of ~70 here,
            # and in the overlapped step the RHT encode runs beside Dgrad, so
            # the step takes the same time either way
            ("quant dY rowwise SR", "hbm", 2.5625 * n_dy,
             lambda: nv.nvfp4_quantize1d_sr(dy, 0, q.qdy.amax, G, SR_SEED, 0, q.qdy.codes,
                                            q.qdy.scales, q.qdy.tensor_scale)),
            ("gemm Dgrad", "mfma", 2.0 * T * F * H, lambda: nv.gemm(q.qdy, q.qw.t(), q.dx)),
            ("quant dY^T RHT SR", "hbm", 2.5625 * n_dy,
             lambda: nv.nvfp4_rht_quantize(dy, RHT_SEED, 1, SR_SEED, 1, q.qdy_t.amax, G,
                                           q.qdy_t.codes, q.qdy_t.scales, q.qdy_t.tensor_scale)),
            ("gemm Wgrad", "mfma", 2.0 * H * F * T, lambda: nv.gemm(q.qdy_t, q.qx_t, q.dw)),
        ]
        del C

    def run(self, events=None):
        for i, (_, _, _, fn) in enumerate(self.ops):
            if events is not None:
                events[i].record()
            fn()
        if events is not None:
            events[len(self.ops)].record()

    def run_cold(self, flush, events, stamps):
        """Each launch on its own, the cache flushed before it, its own HIP
        events around it, and clock stamps around every GEMM."""
        for i, (_, kind, _, fn) in enumerate(self.ops):
            flush()
            if kind == "mfma":
                stamps[i].before()
            events[i][0].record()
            fn()
            events[i][1].record()
            if kind == "mfma":
                stamps[i].after()

    def run_overlapped(self, start=None, end=None):
        """The same launches with the independent chains on a second stream
        (default priority), in the order a forward + backward pass has them:
        W's amax and 2D quantization beside X's, Fprop after both; after dY's
        amaxes, the RHT transpose SR encode beside the rowwise SR encode and
        Dgrad, Wgrad after it.  Each side-stream chain starts behind the
        main stream's earlier work, so steps never overlap each other."""
        if not hasattr(self, "side"):
            self.side = torch.cuda.Stream()
            self.ev = [torch.cuda.Event() for _ in range(4)]
        op = {name: fn for (name, _, _, fn) in self.ops}
        main, side, ev = torch.cuda.current_stream(), self.side, self.ev
        if start is not None:
            start.record(main)
        ev[0].record(main)
        with torch.cuda.stream(side):
            side.wait_event(ev[0])
            op["amax W"]()
            op["quant W 2D RTN +transposed"]()
            ev[1].record(side)
        op["amax X + RHT X"]()
        op["quant X rowwise + X^T RHT RTN"]()
        main.wait_event(ev[1])
        op["gemm Fprop"]()
        op["amax dY + RHT dY"]()
        ev[2].record(main)
        with torch.cuda.stream(side):
            side.wait_event(ev[2])
            op["quant dY^T RHT SR"]()
            ev[3].record(side)
        op["quant dY rowwise SR"]()
        op["gemm Dgrad"]()
        main.wait_event(ev[3])
        op["gemm Wgrad"]()
        if end is not None:
            end.record(main)


C5_SR_SEED, C5_RHT_SEED = 7, 1   # seeds of the whole-tensor oracle comparisons


def oracle_c5(c5, threads, gpu_us):
    """The oracle on the whole 32768x8192 N(0,1) sweep tensor, each
    quantization including its amax pass: 1D RTN on all threads and on one
    thread, 1D SR, 2D RTN and the colwise RHT (RTN) on all threads; codes and
    scales compared with the GPU's, times against the GPU's (cold) ones."""
    import oracle
    x = c5["x"]
    n = x.numel()
    runs = [("1D RTN", 4.5625, (threads, 1), oracle.ROWWISE, {}, "normal 1d RTN incl. amax"),
            ("1D SR", 4.5625, (threads,), oracle.ROWWISE, {"sr_seed": C5_SR_SEED},
             "normal 1d SR incl. amax"),
            ("2D RTN", 4.50390625, (threads,), oracle.TWO_D, {}, "normal 2d RTN incl. amax"),
            ("colwise RHT RTN", 4.5625, (threads,), oracle.COLWISE, {"rht_seed": C5_RHT_SEED},
             "normal col RHT RTN incl. amax")]
    rec = {"workload": "32768x8192 bf16 N(0,1), whole tensor, each quantization incl. its amax",
           "threads": threads}
    for name, bpe, ths, mode, kw, gkey in runs:
        r = {}
        for th in ths:
            oracle.set_num_threads(th)
            t0 = time.perf_counter()
            q = oracle.quantize(x, mode, **kw)
            dt = time.perf_counter() - t0
            r[f"s_{th}_threads"] = round(dt, 3)
            r[f"GB/s_{th}_threads"] = round(bpe * n / dt / 1e9, 3)
        oracle.set_num_threads(threads)
        gc, gs = c5["gpu"][name]
        r["codes_equal_gpu"] = bool(np.array_equal(q.codes, gc) and np.array_equal(q.scales, gs))
        us = gpu_us.get(gkey, {}).get("us")
        if us:
            r["gpu_us"] = us
            r["gpu_speedup_vs_all_threads"] = round(r[f"s_{threads}_threads"] / (us * 1e-6), 1)
        rec[name] = r
        del q
    return rec


def _blas_threads() -> int:
    """Threads of the BLAS the oracle's float64 matmul runs on (0 if unknown)."""
    try:
        from threadpoolctl import threadpool_info
    except ImportError:     # threadpoolctl missing: report the OpenMP count only
        return 0
    n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
    return max(n) if n else 0


def cpu_baseline(x, w, dy, c5=None, gpu_us=None):
    """The oracle, as it stands, on the same host bytes as the GPU:
      * the whole step, timed (the `value`, in the metric's unit): the five
        quantizations of the full tensors, then the three GEMMs through the
        oracle's float64 form (exact decode, float64 library matmul);
      * beside it, the exact int64 GEMM path on a sample of entries (its
        rate, for reference);
      * the 32768x8192 quantizations (oracle_c5)."""
    import oracle
    T, F = x.shape
    H = w.shape[0]
    threads = oracle.num_threads()
    blas = _blas_threads()
    t0 = time.perf_counter()
    ox = oracle.quantize(x, oracle.ROWWISE)
    ox_t = oracle.quantize(x, oracle.COLWISE, rht_seed=RHT_SEED)
    ow = oracle.quantize(w, oracle.TWO_D, with_codes_t=True)
    ody = oracle.quantize(dy, oracle.ROWWISE, sr_seed=SR_SEED)
    ody_t = oracle.quantize(dy, oracle.COLWISE, rht_seed=RHT_SEED, sr_seed=SR_SEED, stream_id=1)
    t_quant = time.perf_counter() - t0
    t1 = time.perf_counter()
    for a, b in [(ox, ow), (ody, ow.transposed()), (ody_t, ox_t)]:
        c = oracle.gemm_f64(a, b, with_bound=False)
        del c
    t_gemm = time.perf_counter() - t1
    full = t_quant + t_gemm
    flops = 3 * 2.0 * T * H * F
    # the exact path's rate on ~3 s of entries
    rng = np.random.default_rng(0)
    n = 4096
    t2 = time.perf_counter()
    oracle.gemm_entries(ox, ow, rng.integers(0, T, n), rng.integers(0, H, n))
    dt = time.perf_counter() - t2
    n2 = int(min(1_000_000, max(n, n * 3.0 / max(dt, 1e-6))))
    t2 = time.perf_counter()
    oracle.gemm_entries(ox, ow, rng.integers(0, T, n2), rng.integers(0, H, n2))
    dt = time.perf_counter() - t2
    # one thread: the Fprop's float64 form on its first 512 rows of X
    rows1 = 512
    ox1 = oracle.quantize(x[:rows1].contiguous(), oracle.ROWWISE)
    t1_thread = None
    try:
        from threadpoolctl import threadpool_limits
        oracle.set_num_threads(1)
        with threadpool_limits(limits=1):
            t3 = time.perf_counter()
            oracle.gemm_f64(ox1, ow, with_bound=False)
            t1_thread = time.perf_counter() - t3
    except ImportError:
        pass
    finally:
        oracle.set_num_threads(threads)
    del ox, ox_t, ow, ody, ody_t, ox1
    out = {"value": flops / full / 1e12, "unit": "TFLOP/s", "cores": max(threads, blas),
           "kind": "oracle",
           "sample": (f"the whole step on the oracle, timed: the 5 quantizations of the full "
                      f"tensors ({t_quant:.1f} s, {threads} OpenMP threads) and the 3 GEMMs "
                      f"through its float64 form ({t_gemm:.1f} s, {blas or threads} BLAS "
                      f"threads); {full:.1f} s per step"),
           "exact_gemm_path": {"TFLOP/s": round(2.0 * n2 * F / dt / 1e12, 5),
                               "sample": f"{n2} exact int64 entries at K={F} ({dt:.1f} s)"}}
    if t1_thread is not None:
        out["gemm_f64_1_thread"] = {
            "TFLOP/s": round(2.0 * rows1 * H * F / t1_thread / 1e12, 4),
            "sample": f"Fprop on the first {rows1} of {T} rows ({t1_thread:.1f} s, 1 thread)"}
    if c5 is not None:
        out["quantize_32768x8192"] = oracle_c5(c5, threads, gpu_us or {})
    return out


def quant_sweep(flush, steps: int = 10, keep_first=False):
    """Quantize-only bandwidth on 32768x8192 tensors (N(0,1) and Student-t,
    generated on the host from seed 0 and copied over): 1D / 2D / colwise
    x RTN / SR, RHT along either axis, with and without the amax pass, and
    MXFP4.  The cache is flushed before every timed launch.  Returns GB/s per
    variant (and, with keep_first, the N(0,1) tensor on the host with the
    GPU's 1D RTN codes and scales, for the oracle's timing on the same bytes)."""
    wl = inputs.sweep_tensors(0)
    out = {}
    kept = None
    valu = quant_valu()
    for dist in ["normal", "t3"]:
        xh = wl.tensors.pop(dist)
        x = xh.cuda()
        n = x.numel()
        q1 = nv.quantize_1d(x)
        q2 = nv.quantize_2d(x)
        qc = nv.quantize_1d(x, nv.NVFP4_COLWISE)
        qr = nv.rht_quantize(x, 1, axis=nv.NVFP4_ROWWISE)
        qm = nv.mx_quantize(x)
        torch.cuda.synchronize()
        if keep_first and kept is None:
            # the GPU's outputs of the whole-tensor quantizations the oracle
            # repeats on the same host bytes (before the timed variants
            # overwrite q1 .. qr)
            qs = nv.quantize_1d(x, sr_seed=C5_SR_SEED)
            qt = nv.rht_quantize(x, C5_RHT_SEED)
            torch.cuda.synchronize()
            host = lambda q: (q.codes.cpu().numpy(), q.scales.cpu().numpy())
            kept = {"x": xh, "gpu": {"1D RTN": host(q1), "1D SR": host(qs), "2D RTN": host(q2),
                                     "colwise RHT RTN": host(qt)}}
            del qs, qt
        del xh
        G, CMP, ROW = nv.NVFP4_AMAX_GIVEN, nv.NVFP4_AMAX_COMPUTE, nv.NVFP4_ROWWISE
        deq = torch.empty(x.shape, dtype=torch.float32, device=x.device)
        variants = [
            ("amax", 2 * n, lambda: nv.nvfp4_amax(x, q1.amax)),
            ("1d RTN encode", 2.5625 * n, lambda: nv.nvfp4_quantize1d_rtn(
                x, 0, q1.amax, G, q1.codes, q1.scales, q1.tensor_scale)),
            ("1d SR encode", 2.5625 * n, lambda: nv.nvfp4_quantize1d_sr(
                x, 0, q1.amax, G, 7, 0, q1.codes, q1.scales, q1.tensor_scale)),
            ("1d RTN incl. amax", 4.5625 * n, lambda: nv.nvfp4_quantize1d_rtn(
                x, 0, q1.amax, CMP, q1.codes, q1.scales, q1.tensor_scale)),
            ("1d SR incl. amax", 4.5625 * n, lambda: nv.nvfp4_quantize1d_sr(
                x, 0, q1.amax, CMP, 7, 0, q1.codes, q1.scales, q1.tensor_scale)),
            ("2d RTN encode", 2.50390625 * n, lambda: nv.nvfp4_quantize2d_rtn(
                x, q2.amax, G, q2.codes, None, q2.scales, None, q2.tensor_scale)),
            ("2d RTN encode +transposed", 3.0078125 * n, lambda: nv.nvfp4_quantize2d_rtn(
                x, q2.amax, G, q2.codes, q2.codes_t, q2.scales, q2.scales_t, q2.tensor_scale)),
            ("2d RTN incl. amax", 4.50390625 * n, lambda: nv.nvfp4_quantize2d_rtn(
                x, q2.amax, CMP, q2.codes, None, q2.scales, None, q2.tensor_scale)),
            ("col RTN encode", 2.5625 * n, lambda: nv.nvfp4_quantize1d_rtn(
                x, 1, qc.amax, G, qc.codes, qc.scales, qc.tensor_scale)),
            ("amax RHT col", 2 * n, lambda: nv.nvfp4_amax_rht(x, 1, qc.amax)),
            ("col RHT RTN encode", 2.5625 * n, lambda: nv.nvfp4_rht_quantize(
                x, 1, 0, 0, 0, qc.amax, G, qc.codes, qc.scales, qc.tensor_scale)),
            ("col RHT SR encode", 2.5625 * n, lambda: nv.nvfp4_rht_quantize(
                x, 1, 1, 7, 0, qc.amax, G, qc.codes, qc.scales, qc.tensor_scale)),
            ("col RHT RTN incl. amax", 4.5625 * n, lambda: nv.nvfp4_rht_quantize(
                x, 1, 0, 0, 0, qc.amax, CMP, qc.codes, qc.scales, qc.tensor_scale)),
            ("col RHT SR incl. amax", 4.5625 * n, lambda: nv.nvfp4_rht_quantize(
                x, 1, 1, 7, 0, qc.amax, CMP, qc.codes, qc.scales, qc.tensor_scale)),
            ("amax RHT row", 2 * n, lambda: nv.nvfp4_amax_rht1d(x, ROW, 1, qr.amax)),
            ("row RHT RTN encode", 2.5625 * n, lambda: nv.nvfp4_rht_quantize1d(
                x, ROW, 1, 0, 0, 0, qr.amax, G, qr.codes, qr.scales, qr.tensor_scale)),
            ("row RHT SR encode", 2.5625 * n, lambda: nv.nvfp4_rht_quantize1d(
                x, ROW, 1, 1, 7, 0, qr.amax, G, qr.codes, qr.scales, qr.tensor_scale)),
            ("row RHT SR incl. amax", 4.5625 * n, lambda: nv.nvfp4_rht_quantize1d(
                x, ROW, 1, 1, 7, 0, qr.amax, CMP, qr.codes, qr.scales, qr.tensor_scale)),
            ("MXFP4 RTN (single pass)", 2.53125 * n, lambda: nv.mxfp4_quantize(
                x, 0, 0, 0, qm.codes, qm.scales)),
            ("MXFP4 SR (single pass)", 2.53125 * n, lambda: nv.mxfp4_quantize(
                x, 1, 7, 0, qm.codes, qm.scales)),
            # codes + scales in, FP32 out
            ("dequantize 1d (FP32 out)", 4.5625 * n, lambda: nv.nvfp4_dequantize(q1, deq)),
        ]
        s = torch.cuda.current_stream()
        for name, nbytes, fn in variants:
            fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                flush()
                a.record(s)
                fn()
                b.record(s)
            s.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            rec = {"us": round(ms * 1e3, 1), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}
            if name in SR_SWEEP_KERNELS:
                # bound by VALU issue: the time the kernel's VALU instructions
                # take at the issue peak, over the measured time (null when the
                # instruction record is stale)
                v8 = (valu or {}).get(SR_SWEEP_KERNELS[name])
                rec["bound"] = "valu"
                rec["valu_frac"] = (round(n * v8 / 8 / VALU_LANE_OPS_PER_S / (ms * 1e-3), 3)
                                    if v8 else None)
            out[f"{dist} {name}"] = rec
        del x, q1, q2, qc, qr, qm, deq
        torch.cuda.empty_cache()
    return (out, kept) if keep_first else out


def _median_ms(fn, reps: int) -> float:
    s = torch.cuda.current_stream()
    fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    s.synchronize()
    for i in range(reps):
        ev[i].record(s)
        fn()
    ev[reps].record(s)
    s.synchronize()
    return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))


def _medians_interleaved(fns: dict, reps: int) -> dict:
    """Median ms of each callable, timed in turn within every repetition so
    that clock drift (the chip warming or cooling after earlier work) weighs
    on all of them alike."""
    s = torch.cuda.current_stream()
    for fn in fns.values():
        fn()
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)] for k in fns}
    s.synchronize()
    for i in range(reps):
        for k, fn in fns.items():
            ev[k][i][0].record(s)
            fn()
            ev[k][i][1].record(s)
    s.synchronize()
    return {k: float(np.median([a.elapsed_time(b) for a, b in ev[k]])) for k in fns}


def quality(step: "Step"):
    """How closely each quantized GEMM tracks the unquantized FP32 product at
    the step's shapes: cosine similarity and relative Frobenius error
    ("NVFP4：让大模型从零预训练跑在4位浮点上", section 4.2's cosine measure), for
    the recipe, the recipe without the Wgrad RHT, RHT also on Fprop and Dgrad
    (an ablation the pages leave unvalidated: "Pretraining Large Language
    Models with NVFP4", limitations paragraph), and MXFP4; on the step's
    gradient and on a Student-t (3 dof) gradient of the same scale."""
    x, w, dy = step.x, step.w, step.dy
    xt, wt = x.t().contiguous(), w.t().contiguous()

    def cmp(got, ref):
        g, r = got.flatten().float(), ref.flatten()
        cos = torch.nn.functional.cosine_similarity(g, r, dim=0)
        rel = torch.linalg.vector_norm(g - r) / torch.linalg.vector_norm(r)
        return {"cos": round(float(cos), 5), "rel_err": round(float(rel), 5)}

    xf, wf = x.float(), w.float()
    out = {}
    yref = xf @ wt.float()
    out["Fprop recipe (X 1D, W 2D)"] = cmp(nv.gemm(nv.quantize_1d(x), nv.quantize_2d(w)), yref)
    row = nv.NVFP4_ROWWISE
    out["Fprop RHT along K (X, W 1D)"] = cmp(
        nv.gemm(nv.rht_quantize(x, RHT_SEED, axis=row), nv.rht_quantize(w, RHT_SEED, axis=row)),
        yref)
    out["Fprop MXFP4"] = cmp(nv.mx_gemm(nv.mx_quantize(x), nv.mx_quantize(w)), yref)
    del yref
    g = torch.Generator(device=dy.device).manual_seed(7)
    z = torch.randn(4, *dy.shape, generator=g, device=dy.device)
    t3 = (z[0] / torch.sqrt((z[1] ** 2 + z[2] ** 2 + z[3] ** 2) / 3)).mul_(float(dy.float().std()))
    del z
    for tag, d in [("", dy), (" t3", t3.to(torch.bfloat16))]:
        dt = d.t().contiguous()
        df = d.float()
        dxref = df @ wf
        qw = nv.quantize_2d(w)
        out[f"Dgrad recipe (dY 1D SR){tag}"] = cmp(
            nv.gemm(nv.quantize_1d(d, sr_seed=SR_SEED), qw.t()), dxref)
        out[f"Dgrad RHT along K (dY SR, W 1D){tag}"] = cmp(
            nv.gemm(nv.rht_quantize(d, RHT_SEED, sr_seed=SR_SEED, axis=row),
                    nv.rht_quantize(w, RHT_SEED)), dxref)
        out[f"Dgrad MXFP4 SR{tag}"] = cmp(
            nv.mx_gemm(nv.mx_quantize(d, SR_SEED), nv.mx_quantize(wt)), dxref)
        del dxref, qw
        dwref = dt.float() @ xf
        out[f"Wgrad recipe (RHT, dY SR){tag}"] = cmp(
            nv.gemm(nv.rht_quantize(d, RHT_SEED, sr_seed=SR_SEED, stream_id=1),
                    nv.rht_quantize(x, RHT_SEED)), dwref)
        out[f"Wgrad no RHT (dY SR){tag}"] = cmp(
            nv.gemm(nv.quantize_1d(d, nv.NVFP4_COLWISE, sr_seed=SR_SEED, stream_id=1),
                    nv.quantize_1d(x, nv.NVFP4_COLWISE)), dwref)
        out[f"Wgrad MXFP4 SR{tag}"] = cmp(
            nv.mx_gemm(nv.mx_quantize(dt, SR_SEED), nv.mx_quantize(xt)), dwref)
        del dwref, dt, df
    del t3, xt, wt, xf, wf
    torch.cuda.empty_cache()
    return out


def fused_epilogue(step: "Step", reps: int):
    """The fused BF16 + amax epilogue vs the FP32 GEMM followed by the separate
    amax read of C that the next layer's quantization needs, at the Fprop and
    Dgrad shapes.  With its workspace the BF16 path cuts the last round's tiles
    along K as the FP32 path does (Fprop: 640 tiles, 2.5 rounds); "no workspace"
    times it with half-width tiles there instead.  The variants are timed in
    turn within each repetition."""
    out = {}
    for name, qa, qb, c32 in [("Fprop", step.qx, step.qw, step.y),
                              ("Dgrad", step.qdy, step.qw.t(), step.dx)]:
        cb = torch.empty(qa.rows, qb.rows, dtype=torch.bfloat16, device=step.x.device)
        am = torch.empty(1, dtype=torch.float32, device=step.x.device)
        ws = nv.gemm_bf16_workspace(qa.rows, qb.rows, qa.k, step.x.device)
        fns = {"fused": lambda: nv.nvfp4_gemm_bf16(qa, qb, cb, cb.stride(0), am, ws),
               "plain": lambda: nv.gemm(qa, qb, c32),
               "scan": lambda: nv.nvfp4_amax(cb, am)}
        if ws is not None:
            fns["no_ws"] = lambda: nv.nvfp4_gemm_bf16(qa, qb, cb, cb.stride(0), am)
        t = _medians_interleaved(fns, reps)
        fused, plain, scan = t["fused"], t["plain"], t["scan"]
        no_ws = t.get("no_ws", fused)
        fl = 2.0 * qa.rows * qb.rows * qa.k
        out[name] = {"fused bf16 + amax us": round(fused * 1e3, 1),
                     "fused, no workspace us": round(no_ws * 1e3, 1),
                     "fp32 gemm us": round(plain * 1e3, 1),
                     "separate amax of C us": round(scan * 1e3, 1),
                     "fused TFLOP/s": round(fl / (fused * 1e-3) / 1e12, 1),
                     "saved us": round((plain + scan - fused) * 1e3, 1)}
        del cb, ws
    return out


def mx_comparison(step: "Step", reps: int):
    """The same three GEMMs with MXFP4 operands on the scaled FP4 matrix cores
    (the format the NVFP4 pages compare against), and the relative
    quantization error of both formats on the step's tensors."""
    x, w, dy = step.x, step.w, step.dy
    T, F = x.shape
    H = w.shape[0]
    qx, qw, qdy = nv.mx_quantize(x), nv.mx_quantize(w), nv.mx_quantize(dy)
    wt, dyt, xt = w.t().contiguous(), dy.t().contiguous(), x.t().contiguous()
    qwt, qdyt, qxt = nv.mx_quantize(wt), nv.mx_quantize(dyt, sr_seed=SR_SEED), nv.mx_quantize(xt)
    out = {}
    for name, a, b, c in [("Fprop", qx, qw, step.y), ("Dgrad", qdy, qwt, step.dx),
                          ("Wgrad", qdyt, qxt, step.dw)]:
        ms = _median_ms(lambda: nv.mx_gemm(a, b, c), reps)
        tf = 2.0 * a.rows * b.rows * a.k / (ms * 1e-3) / 1e12
        out[f"gemm {name} {a.rows}x{b.rows}x{a.k}"] = {
            "us": round(ms * 1e3, 1), "TFLOP/s": round(tf, 1),
            "frac_fp4_peak": round(tf / MFMA_FP4_PEAK_TFLOPS, 3)}
    n = x.numel()
    ms = _median_ms(lambda: nv.mxfp4_quantize(x, 0, 0, 0, qx.codes, qx.scales), reps)
    out["quantize X RTN (single pass)"] = {"us": round(ms * 1e3, 1),
                                           "GB/s": round(2.53125 * n / (ms * 1e-3) / 1e9, 1)}

    def rel_err(deq, ref):
        r = ref.float()
        return round(float(torch.linalg.vector_norm(deq - r) / torch.linalg.vector_norm(r)), 5)
    out["relative quantization error"] = {
        "X (NVFP4 1D RTN | MXFP4 RTN)": [rel_err(nv.dequantize(step.qx), x),
                                         rel_err(nv.mx_dequantize(qx), x)],
        "W (NVFP4 2D RTN | MXFP4 RTN)": [rel_err(nv.dequantize(step.qw), w),
                                         rel_err(nv.mx_dequantize(qw), w)],
        "dY (NVFP4 1D RTN | MXFP4 RTN)": [rel_err(nv.dequantize(nv.quantize_1d(dy)), dy),
                                          rel_err(nv.mx_dequantize(qdy), dy)],
        "dY (NVFP4 1D SR | MXFP4 SR)": [rel_err(nv.dequantize(step.qdy), dy),
                                        rel_err(nv.mx_dequantize(nv.mx_quantize(dy, SR_SEED)), dy)],
    }
    del qx, qw, qdy, qwt, qdyt, qxt, wt, dyt, xt
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-mx", action="store_true", help="skip the MXFP4 comparison")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the cosine / error comparison with FP32 products")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step and stop: no MXFP4, epilogue, quality, sweep or CPU "
                         "sections (for profiler runs, whose per-kernel averages then cover "
                         "the step's launches alone)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="run only the 32768x8192 quantize sweep and print its JSON (for "
                         "profiler runs over the quantizer kernels on large tensors)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run the plain 1 GiB device copy k_copy (3 launches), the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.step_only:
        args.no_mx = args.no_quality = args.no_sweep = args.no_cpu_baseline = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(rerun with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    nv.load_library()

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            nv.probe_copy(src, dst)
        torch.cuda.synchronize()
        log("copy calibration: 3 x k_copy of 1 GiB (read 1 GiB + write 1 GiB each)")
        del src, dst
    if args.sweep_only:
        log("quantize sweep 32768x8192")
        print(json.dumps({"quantize_sweep_32768x8192": quant_sweep(Flush(),
                                                                    max(args.steps, 2))}),
              flush=True)
        return

    log("generating inputs (host, seeded)")
    wl = inputs.ffn_down(args.seed, TOKENS, HIDDEN, FFN)
    xh, wh, dyh = wl.tensors["X"], wl.tensors["W"], wl.tensors["dY"]
    dev = torch.device("cuda")
    x, w, dy = xh.to(dev), wh.to(dev), dyh.to(dev)
    step = Step(x, w, dy)

    flush = Flush()
    log("hbm copy peak")
    hbm_copy = copy_peak()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    nops = len(step.ops)
    # serial pass: the launches back to back, events between them (warm caches)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nops + 1)]
           for _ in range(args.steps)]
    log(f"timing {args.steps} serial steps")
    torch.cuda.synchronize()
    for k in range(args.steps):
        step.run(evs[k])
    torch.cuda.synchronize()
    per_op_warm = np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(nops)]
                            for k in range(args.steps)])  # ms
    serial_ms = float(np.median([evs[k][0].elapsed_time(evs[k][nops])
                                 for k in range(args.steps)]))
    # cold pass: every launch timed on its own after a cache flush, GEMM clocks
    log(f"timing {args.steps} cold-cache passes")
    gemm_idx = [i for i, o in enumerate(step.ops) if o[1] == "mfma"]
    stamps = {i: nv.ClockStamps() for i in gemm_idx}
    clocks = {i: [] for i in gemm_idx}
    cev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(nops)] for _ in range(args.steps)]
    for k in range(args.steps):
        step.run_cold(flush, cev[k], stamps)
        for i in gemm_idx:
            clocks[i].append(stamps[i].ghz())
    torch.cuda.synchronize()
    per_op = np.array([[cev[k][i][0].elapsed_time(cev[k][i][1]) for i in range(nops)]
                       for k in range(args.steps)])  # ms
    # the step as a framework would run it: independent chains on two streams
    log(f"timing {args.steps} overlapped steps")
    for _ in range(max(args.warmup, 1)):
        step.run_overlapped()
    oev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step.run_overlapped(*oev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = float(np.median([a.elapsed_time(b) for a, b in oev]))
    gemm_flops = sum(a for (_, kind, a, _) in step.ops if kind == "mfma")
    value = gemm_flops / (step_ms * 1e-3) / 1e12

    kernels = {}
    for i, (name, kind, amount, _) in enumerate(step.ops):
        ms = float(np.median(per_op[:, i]))
        rec = {"us": round(ms * 1e3, 1), "us_warm": round(float(np.median(per_op_warm[:, i])) * 1e3, 1)}
        if kind == "hbm":
            gbs = amount / (ms * 1e-3) / 1e9
            rec.update({"GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 3),
                        "frac_copy": round(gbs / hbm_copy["GB/s"], 3)})
        else:
            tf = amount / (ms * 1e-3) / 1e12
            rec.update({"TFLOP/s": round(tf, 1), "frac_mfma": round(tf / MFMA_F16_PEAK_TFLOPS, 3),
                        "clock_GHz": round(float(np.median(clocks[i])), 3)})
        kernels[name] = rec
    gemm_ms_mean = float(per_op[:, gemm_idx].mean())
    gemm_flops_launch = gemm_flops / len(gemm_idx)
    achieved = gemm_flops_launch / (gemm_ms_mean * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "k_gemm_dma (Fprop, Dgrad, Wgrad launches)",
                "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": gemm_traffic(),
                "launch_us_mean": round(gemm_ms_mean * 1e3, 1),
                "clock_GHz_median": round(float(np.median([c for i in gemm_idx
                                                           for c in clocks[i]])), 3)}
    quant_idx = [i for i in range(nops) if i not in gemm_idx]
    quant_ms = float(np.median(per_op[:, quant_idx].sum(axis=1)))
    quant_bytes = sum(a for (_, kind, a, _) in step.ops if kind == "hbm")

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "ms_per_step_serial": round(serial_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 operands, fp16 mfma, fp32 accumulate", "data": "synthetic",
        "config": {"workload": "NVFP4 linear fwd+bwd triple, FFN down-projection: "
                               "X 8192x20480, W 5120x20480, dY 8192x5120 (bf16, seed 0)",
                   "tokens": TOKENS, "in_features": FFN, "out_features": HIDDEN,
                   "gemms": "Fprop 8192x5120x20480, Dgrad 8192x20480x5120, "
                            "Wgrad 5120x20480x8192",
                   "quantization": "X 1D RTN, W 2D RTN, dY 1D SR, Wgrad inputs RHT16 "
                                   "(dY SR, X RTN)"},
        "timing": "medians of HIP events on the launch stream; `value` and ms_per_step from the "
                  "overlapped step (warm caches, as in training); per-kernel us / GB/s from "
                  "launches timed one by one after a 1 GiB cache-flush write (us_warm: the "
                  "serial pass without the flush); roofline.achieved from the mean GEMM launch",
        "gemm_tflops": round(achieved, 1),
        "quantize_gbs": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "quantize_ms_per_step": round(quant_ms, 4),
        "hbm_copy_peak": hbm_copy,
        "kernels": kernels,
        "roofline": roofline,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_mx:
        log("MXFP4 comparison")
        result["mxfp4_comparison"] = mx_comparison(step, max(args.steps, 5))
    if not args.step_only:
        log("fused epilogue")
        result["fused_epilogue"] = fused_epilogue(step, max(args.steps, 5))
    if not args.step_only:
        log("matrix-core ceiling (probe)")
        ceil = {}
        for mode, name in ((nv.PROBE_ZEROS, "zeros"), (nv.PROBE_NVFP4_LIKE, "nvfp4-like"),
                           (nv.PROBE_UNIFORM, "uniform fp16")):
            tf, ghz = nv.probe_mfma(mode, 200000)   # ~50 ms: the sustained clock
            ceil[name] = {"TFLOP/s": round(tf, 1), "clock_GHz": round(ghz, 3)}
        ceil["gemm_frac_of_nvfp4_like"] = round(achieved / ceil["nvfp4-like"]["TFLOP/s"], 4)
        result["mfma_ceiling"] = ceil
    if not args.no_quality:
        log("quality (cosine vs FP32 products)")
        result["quality"] = quality(step)
    c5 = None
    if not args.no_sweep:
        log("quantize sweep 32768x8192")
        del step, x, w, dy
        torch.cuda.empty_cache()
        sweep, c5 = quant_sweep(flush, keep_first=not args.no_cpu_baseline)
        result["quantize_sweep_32768x8192"] = sweep
        result["quantize_sweep_bounds"] = {
            "hbm": "frac = algorithmic bytes / time / 8 TB/s",
            "valu": "SR encodes: valu_frac = VALU lane-instructions (rocprofv3 SQ_INSTS_VALU "
                    "per 8 elements, profiles/quantize_valu.json) / time / peak; peak "
                    f"{VALU_LANE_OPS_PER_S:.4g} lane-instructions/s = 1024 SIMDs x 16 lanes a "
                    "cycle x 2.4 GHz"}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on the same host bytes")
        result["cpu_baseline"] = cpu_baseline(xh, wh, dyh, c5,
                                              result.get("quantize_sweep_32768x8192", {}))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
