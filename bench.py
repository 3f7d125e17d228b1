#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

Default workload (``wgrad_8192x5120``): one step = quantise dY (8192x5120 bf16,
Laplace(0,1e-3)) column-wise with the 16x16 RHT and stochastic rounding,
quantise X (8192x5120, N(0,1)) column-wise with the RHT and RTN, and the NVFP4
weight-gradient GEMM dW = dY^T X (5120x5120, K = 8192, fp32 out).  This is the
workload on which both halves of the metric (quantise GB/s, Wgrad GEMM
TFLOP/s) are quoted.  Other workloads (``--workload``): ``act_8192x5120``
(row + column quantise of an activation), ``weight_5120x20480`` (2D + 2D_T),
``tiny_256``, ``linear_step_16384`` (Fprop/Dgrad/Wgrad of a 5120/20480
two-layer FFN over 16384 tokens) and ``mx_wgrad_8192x5120`` (the same Wgrad
step in MXFP4, the earlier microscaling format the page compares NVFP4 with:
single-pass quantise of dY and X along tokens, GEMM on the block-scaled FP4
MFMA; its roofline is against the FP4 matrix peak).

Prints ONE JSON line.  ``value`` is whole-step throughput (GEMM flops of the
step over the wall time per step, inputs resident in HBM).  In the timed steps
only the dominant call is bracketed by HIP events (on the stream the library
launches on), which gives the roofline's kernel time; the other per-call times
come from further steps after the timed region with every call bracketed, as
each event pair adds GPU time to a step.  The ``roofline`` object is for the
dominant kernel; ``cpu_baseline`` times the CPU oracle on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def qbytes(rows, cols, outs=1):
    """Algorithmic bytes of one quantise call: one bf16 read + codes + scales of each output."""
    n = rows * cols
    return 2 * n + outs * (n // 2 + n // 16)


def code_only(src: str) -> str:
    """C/HIP source without comments and whitespace (string literals kept)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c == '"':
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def source_hash(*names):
    """Hash of the code (comments and whitespace excluded) of the named
    sources: counter profiles taken on other code are not reused."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "nvfp4_bit_quantization_amd", "csrc", n)) as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary for this
    kernel, if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, kernel_tag + "_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_hash:\s*(\w+)", txt)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != src_hash:
        return None
    return float(t.group(1))


class Timer:
    """HIP events around library calls on the current stream.  With `live`
    given, only the calls named there are bracketed (the others just run):
    every event pair adds a few microseconds of GPU time to a step."""

    def __init__(self, live=None):
        self.marks = {}
        self.live = live

    def run(self, name, fn):
        import torch
        if self.live is not None and name not in self.live:
            fn()
            return
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.marks.setdefault(name, []).append((s, e))

    def times(self, name):
        return [s.elapsed_time(e) for s, e in self.marks[name]]

    def ms(self, name):
        return float(np.mean(self.times(name)))

    def stats(self, name):
        """mean, median, min and max (ms) of the bracketed calls of `name`."""
        t = np.array(self.times(name))
        return dict(ms=round(float(t.mean()), 4), ms_median=round(float(np.median(t)), 4),
                    ms_min=round(float(t.min()), 4), ms_max=round(float(t.max()), 4), n=int(t.size))


class GpuSampler:
    """Samples, from a host thread while the timed steps run, the GPU's board
    power (hwmon power1_input, with its cap power1_cap) and its current
    graphics-clock DPM level (pp_dpm_sclk) from sysfs: plain file reads, no
    GPU work.  Fields are None where the files are absent."""

    def __init__(self, period_s=0.0005):
        import glob
        import threading
        cards = sorted(d for d in glob.glob("/sys/class/drm/card*/device") if os.path.exists(d + "/pp_dpm_sclk"))
        self.dev = cards[0] if len(cards) == 1 else None
        hw = sorted(glob.glob(self.dev + "/hwmon/hwmon*")) if self.dev else []
        self.hw = hw[0] if hw else None
        self.period = period_s
        self.power, self.sclk = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    def _run(self):
        while not self._stop.is_set():
            if self.hw:
                v = self._read(self.hw + "/power1_input")
                if v and v.strip().isdigit():
                    self.power.append(int(v) / 1e6)  # microwatts -> W
            if self.dev:
                v = self._read(self.dev + "/pp_dpm_sclk")
                m = re.search(r"(\d+)\s*[Mm]hz\s*\*", v or "")
                if m:
                    self.sclk.append(int(m.group(1)))
            time.sleep(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        cap = self._read(self.hw + "/power1_cap") if self.hw else None
        out = dict(samples=len(self.power),
                   power_w_mean=round(float(np.mean(self.power)), 1) if self.power else None,
                   power_w_max=round(float(np.max(self.power)), 1) if self.power else None,
                   power_cap_w=round(int(cap) / 1e6, 1) if cap and cap.strip().isdigit() else None,
                   sclk_dpm_mhz=sorted(set(self.sclk)) if self.sclk else None,
                   source="sysfs hwmon power1_input/power1_cap, pp_dpm_sclk (current DPM level), sampled "
                          "every ~%.1f ms during the timed steps" % (self.period * 1e3))
        return out


# ---------------------------------------------------------------------------
# workloads: each returns (step(timer), info dict)
# ---------------------------------------------------------------------------
def setup_wgrad(nv, syn, tokens=8192, hidden=5120):
    import torch
    dy_bits, x_bits = syn.wgrad_8192x5120(tokens, hidden)
    dy, x = dev_bf16(dy_bits), dev_bf16(x_bits)
    ws, gws = nv.new_workspace(jobs=2), nv.new_gemm_workspace()
    s_dy = [nv.QuantSpec.of("col", "sr", True, 1234, 1234)]
    s_x = [nv.QuantSpec.of("col", "rtn", True, 0, 1234)]
    q_dy = [nv.empty_qtensor(hidden, tokens, nv.SCALE_1D16, rht=1)]
    q_x = [nv.empty_qtensor(hidden, tokens, nv.SCALE_1D16, rht=1)]
    c = torch.empty((hidden, hidden), dtype=torch.float32, device="cuda")
    flops = 2.0 * hidden * hidden * tokens
    jobs = [(dy, s_dy, q_dy), (x, s_x, q_x)]

    def step(t: Timer):
        # both Wgrad operands in one batch: one amax launch, one quantise launch
        t.run("quantize_dY_X", lambda: nv.nvfp4_quantize_batch(jobs, ws))
        t.run("gemm_wgrad", lambda: nv.nvfp4_gemm(q_dy[0], q_x[0], c, gws))

    info = dict(flops=flops, calls={
        "quantize_dY_X": dict(kind="quantize", bytes=2 * qbytes(tokens, hidden)),
        "gemm_wgrad": dict(kind="gemm", flops=flops, M=hidden, N=hidden, K=tokens)},
        dominant="gemm_wgrad", config=dict(workload="wgrad_8192x5120", tokens=tokens, hidden=hidden,
                                           quantize="dY col1D+RHT+SR(seed 1234) and X col1D+RHT+RTN, RHT seed 1234, "
                                                    "as one nvfp4_quantize_batch call",
                                           gemm="dW = dY^T X, M=N=%d, K=%d, fp32 out" % (hidden, tokens)))
    return step, info


def setup_act(nv, syn):
    bits = syn.act_8192x5120()
    x = dev_bf16(bits)
    ws = nv.new_workspace()
    specs = [nv.QuantSpec.of("row"), nv.QuantSpec.of("col")]
    outs = [nv.empty_qtensor(8192, 5120, 0), nv.empty_qtensor(5120, 8192, 0)]

    def step(t):
        t.run("quantize_act_row_col", lambda: nv.nvfp4_quantize(x, specs, outs, ws))

    return step, dict(flops=0.0, calls={"quantize_act_row_col": dict(kind="quantize", bytes=qbytes(8192, 5120, 2))},
                      dominant="quantize_act_row_col",
                      config=dict(workload="act_8192x5120", quantize="row1D + col1D RTN from one read"))


def setup_weight(nv, syn):
    bits = syn.weight_5120x20480()
    x = dev_bf16(bits)
    ws = nv.new_workspace()
    specs = [nv.QuantSpec.of("2d"), nv.QuantSpec.of("2d_t")]
    outs = [nv.empty_qtensor(5120, 20480, 1), nv.empty_qtensor(20480, 5120, 1)]
    n = 5120 * 20480
    b = 2 * n + 2 * (n // 2 + n // 256)

    def step(t):
        t.run("quantize_weight_2d", lambda: nv.nvfp4_quantize(x, specs, outs, ws))

    return step, dict(flops=0.0, calls={"quantize_weight_2d": dict(kind="quantize", bytes=b)},
                      dominant="quantize_weight_2d",
                      config=dict(workload="weight_5120x20480", quantize="2D 16x16 RTN + transposed copy"))


def setup_tiny(nv, syn):
    bits = syn.tiny_256()
    x = dev_bf16(bits)
    ws = nv.new_workspace()
    specs = [nv.QuantSpec.of("row")]
    outs = [nv.empty_qtensor(256, 256, 0)]
    import torch
    y = torch.empty((256, 256), dtype=torch.float32, device="cuda")

    def step(t):
        t.run("quantize_tiny", lambda: nv.nvfp4_quantize(x, specs, outs, ws))
        t.run("dequantize_tiny", lambda: nv.nvfp4_dequantize(outs[0], y))

    return step, dict(flops=0.0, calls={"quantize_tiny": dict(kind="quantize", bytes=qbytes(256, 256)),
                                        "dequantize_tiny": dict(kind="quantize", bytes=256 * 256 * (4 + 0.5625))},
                      dominant="quantize_tiny", config=dict(workload="tiny_256"))


def setup_linear(nv, syn, tokens=16384, hidden=5120, ffn=20480):
    import torch
    d = syn.linear_step_16384(tokens, hidden, ffn)
    X, W1, W2, dY = (dev_bf16(d[k]) for k in ("X", "W1", "W2", "dY"))
    del d
    ws, gws = nv.new_workspace(), nv.new_gemm_workspace()
    bf, f32 = torch.bfloat16, torch.float32
    H = torch.empty((tokens, ffn), dtype=bf, device="cuda")
    Y = torch.empty((tokens, hidden), dtype=bf, device="cuda")
    dH = torch.empty((tokens, ffn), dtype=bf, device="cuda")
    dX = torch.empty((tokens, hidden), dtype=bf, device="cuda")
    dW1 = torch.empty((ffn, hidden), dtype=f32, device="cuda")
    dW2 = torch.empty((hidden, ffn), dtype=f32, device="cuda")
    E = nv.empty_qtensor
    qX = [E(tokens, hidden, 0), E(hidden, tokens, 0, rht=1)]
    qW1 = [E(ffn, hidden, 1), E(hidden, ffn, 1)]
    qH = [E(tokens, ffn, 0), E(ffn, tokens, 0, rht=1)]
    qW2 = [E(hidden, ffn, 1), E(ffn, hidden, 1)]
    qdY = [E(tokens, hidden, 0), E(hidden, tokens, 0, rht=1)]
    qdH = [E(tokens, ffn, 0), E(ffn, tokens, 0, rht=1)]
    S = nv.QuantSpec.of
    sX = [S("row"), S("col", "rtn", True, 0, 4321)]
    sW = [S("2d"), S("2d_t")]
    sdY = [S("row", "sr", False, 1234), S("col", "sr", True, 1235, 4321)]
    # H and dH are GEMM outputs: their GEMMs produce the maxima of both of
    # their quantisations (producer-fused amax), so those calls skip the amax pass
    sH = [S("row", amax_given=True), S("col", "rtn", True, 0, 4321, amax_given=True)]
    sdH = [S("row", "sr", False, 1236, amax_given=True), S("col", "sr", True, 1237, 4321, amax_given=True)]
    amax4 = torch.zeros(4, dtype=f32, device="cuda")
    qH[0].amax, qH[1].amax, qdH[0].amax, qdH[1].amax = amax4[0:1], amax4[1:2], amax4[2:3], amax4[3:4]
    g = 2.0 * tokens * ffn * hidden

    def fprop_h():
        amax4.zero_()
        nv.nvfp4_gemm_amax(qX[0], qW1[0], H, qH[0].amax, qH[1].amax, 4321, gws)

    def step(t):
        t.run("q_X", lambda: nv.nvfp4_quantize(X, sX, qX, ws))
        t.run("q_W1", lambda: nv.nvfp4_quantize(W1, sW, qW1, ws))
        t.run("fprop_H", fprop_h)
        t.run("q_H", lambda: nv.nvfp4_quantize(H, sH, qH, ws))
        t.run("q_W2", lambda: nv.nvfp4_quantize(W2, sW, qW2, ws))
        t.run("fprop_Y", lambda: nv.nvfp4_gemm(qH[0], qW2[0], Y, gws))
        t.run("q_dY", lambda: nv.nvfp4_quantize(dY, sdY, qdY, ws))
        t.run("dgrad_dH", lambda: nv.nvfp4_gemm_amax(qdY[0], qW2[1], dH, qdH[0].amax, qdH[1].amax, 4321, gws))
        t.run("q_dH", lambda: nv.nvfp4_quantize(dH, sdH, qdH, ws))
        t.run("dgrad_dX", lambda: nv.nvfp4_gemm(qdH[0], qW1[1], dX, gws))
        t.run("wgrad_dW2", lambda: nv.nvfp4_gemm(qdY[1], qH[1], dW2, gws))
        t.run("wgrad_dW1", lambda: nv.nvfp4_gemm(qdH[1], qX[1], dW1, gws))

    calls = {
        "q_X": dict(kind="quantize", bytes=qbytes(tokens, hidden, 2)),
        "q_W1": dict(kind="quantize", bytes=2 * ffn * hidden + 2 * (ffn * hidden // 2 + ffn * hidden // 256)),
        "fprop_H": dict(kind="gemm", flops=g), "q_H": dict(kind="quantize", bytes=qbytes(tokens, ffn, 2)),
        "q_W2": dict(kind="quantize", bytes=2 * ffn * hidden + 2 * (ffn * hidden // 2 + ffn * hidden // 256)),
        "fprop_Y": dict(kind="gemm", flops=g), "q_dY": dict(kind="quantize", bytes=qbytes(tokens, hidden, 2)),
        "dgrad_dH": dict(kind="gemm", flops=g), "q_dH": dict(kind="quantize", bytes=qbytes(tokens, ffn, 2)),
        "dgrad_dX": dict(kind="gemm", flops=g), "wgrad_dW2": dict(kind="gemm", flops=g, M=hidden, N=ffn, K=tokens),
        "wgrad_dW1": dict(kind="gemm", flops=g)}
    # dW2 (1600 256x256 tiles: 6.25 rounds on 256 CUs) runs as stream-K
    return step, dict(flops=6 * g, calls=calls, dominant="wgrad_dW2", kernel="gemm_streamk_kernel",
                      config=dict(workload="linear_step_16384", tokens=tokens, hidden=hidden, ffn=ffn,
                                  step="Fprop H,Y; Dgrad dH,dX; Wgrad dW2,dW1; 6 quantise calls; "
                                       "H and dH maxima fused into their GEMMs"))


def setup_mx_wgrad(nv, syn, tokens=8192, hidden=5120):
    import torch
    dy_bits, x_bits = syn.wgrad_8192x5120(tokens, hidden)
    dy, x = dev_bf16(dy_bits), dev_bf16(x_bits)
    q_dy, q_x = nv.empty_mxtensor(hidden, tokens), nv.empty_mxtensor(hidden, tokens)
    c = torch.empty((hidden, hidden), dtype=torch.float32, device="cuda")
    flops = 2.0 * hidden * hidden * tokens
    mxbytes = tokens * hidden * 2 + tokens * hidden // 2 + tokens * hidden // 32

    def step(t: Timer):
        t.run("quantize_dY", lambda: nv.mxfp4_quantize(dy, nv.COL_1D, q_dy))
        t.run("quantize_X", lambda: nv.mxfp4_quantize(x, nv.COL_1D, q_x))
        t.run("gemm_wgrad", lambda: nv.mxfp4_gemm(q_dy, q_x, c))

    info = dict(flops=flops, calls={
        "quantize_dY": dict(kind="quantize", bytes=mxbytes),
        "quantize_X": dict(kind="quantize", bytes=mxbytes),
        "gemm_wgrad": dict(kind="gemm", flops=flops, peak=MFMA_FP4_PEAK_TFLOPS, M=hidden, N=hidden, K=tokens)},
        dominant="gemm_wgrad", kernel="mx_gemm_fast_kernel",
        sources=("mxfp4.hip", "gemm_device.hpp", "nvfp4_kernels.hpp"),
        dtype="mxfp4 operands (E2M1, E8M0 per 32); fp32 quantise math; fp4 MFMA with block scales, fp32 accumulate",
        config=dict(workload="mx_wgrad_8192x5120", tokens=tokens, hidden=hidden,
                    quantize="dY, X MXFP4 along tokens (OCP MX: 32-element blocks, E8M0 scale, RNE), one pass each",
                    gemm="dW = dY^T X, M=N=%d, K=%d, fp32 out, block-scaled FP4 MFMA" % (hidden, tokens)))
    return step, info


WORKLOADS = {"wgrad_8192x5120": setup_wgrad, "act_8192x5120": setup_act, "weight_5120x20480": setup_weight,
             "tiny_256": setup_tiny, "linear_step_16384": setup_linear, "mx_wgrad_8192x5120": setup_mx_wgrad}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the workload
# ---------------------------------------------------------------------------
def library_gemm(M: int, N: int, K: int, reps: int = 30):
    """torch.matmul (hipBLASLt) in bf16 on random [M][K] x [N][K]^T operands:
    TFLOP/s and ms per call, HIP events around `reps` back-to-back calls."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(5):
        a @ b.t()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        a @ b.t()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return dict(tflops=round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1), ms=round(ms, 4), shape="%dx%dx%d" % (M, N, K),
                what="torch.matmul bf16 (hipBLASLt), random operands, A [M][K] x B[N][K]^T")


def host_info():
    """The host the CPU baseline ran on: CPU model, threads this process may
    use, and the BLAS numpy calls for the oracle's GEMM."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        threads = os.cpu_count()
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = "%s %s" % (b.get("name", "?"), b.get("version", ""))
        try:
            from threadpoolctl import threadpool_info
            libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
            if libs:
                blas += " (%s, %s threads)" % (libs[0].get("internal_api"), libs[0].get("num_threads"))
        except Exception:  # pragma: no cover
            pass
    except Exception:  # pragma: no cover
        pass
    return dict(cpu_model=model, threads=threads, blas=blas.strip() if blas else None)


def median_time(fn, reps: int = 5) -> float:
    """Median wall time (s) of `reps` calls of fn after one untimed call."""
    fn()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def one_thread(fn) -> float:
    """Wall time of fn() with the oracle's parallel loops and the BLAS on one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    n = oracle.threads()
    oracle.set_threads(1)
    try:
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            fn()
            return time.perf_counter() - t0
    finally:
        oracle.set_threads(n)


def cpu_baseline(workload: str, syn):
    """The oracle timed on the host: on all threads (``value``) and on one
    (``value_1thread``; its GEMM timed on a row sample and scaled)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    qthreads = oracle.threads()
    if workload == "wgrad_8192x5120":
        dy, xx = syn.wgrad_8192x5120()
        qa = oracle.quantize(dy, "col", "sr", True, 1234, 1234)
        qb = oracle.quantize(xx, "col", "rtn", True, 0, 1234)
        tq = median_time(lambda: (oracle.quantize(dy, "col", "sr", True, 1234, 1234),
                                  oracle.quantize(xx, "col", "rtn", True, 0, 1234)))
        tg = median_time(lambda: oracle.gemm_f64(qa, qb))
        flops = 2.0 * 5120 * 5120 * 8192
        tq1 = one_thread(lambda: (oracle.quantize(dy, "col", "sr", True, 1234, 1234),
                                  oracle.quantize(xx, "col", "rtn", True, 0, 1234)))
        tg1 = 8 * one_thread(lambda: oracle.gemm_f64(qa, qb, rows_a=np.arange(640)))
        return dict(value=flops / (tq + tg) / 1e12, unit="TFLOP/s", cores=max(qthreads, blas_threads),
                    kind="oracle", value_1thread=flops / (tq1 + tg1) / 1e12, host=host_info(),
                    sample="the whole Wgrad workload (dY, X 8192x5120), medians of 5 runs after one warm-up: "
                           "C oracle quantise (col+RHT, SR/RTN; %d threads, %.2f s) + binary64 GEMM "
                           "5120x5120x8192 (BLAS, %d threads, %.2f s); 1 thread, one run: quantise %.2f s, "
                           "GEMM 8 x the time of 640 rows of C, %.2f s"
                           % (qthreads, tq, blas_threads, tg, tq1, tg1))
    if workload == "mx_wgrad_8192x5120":
        dy, xx = syn.wgrad_8192x5120()
        t0 = time.perf_counter()
        qa = oracle.mx_quantize(dy, "col")
        qb = oracle.mx_quantize(xx, "col")
        t1 = time.perf_counter()
        oracle.mx_gemm_f64(qa, qb)
        t2 = time.perf_counter()
        flops = 2.0 * 5120 * 5120 * 8192
        tq1 = one_thread(lambda: (oracle.mx_quantize(dy, "col"), oracle.mx_quantize(xx, "col")))
        return dict(value=flops / (t2 - t0) / 1e12, unit="TFLOP/s", cores=max(qthreads, blas_threads),
                    kind="oracle", value_1thread=flops / (tq1 + (t2 - t1) * blas_threads) / 1e12,
                    sample="the whole MXFP4 Wgrad workload (dY, X 8192x5120): C oracle MX quantise (%d threads, "
                           "%.2f s) + binary64 GEMM 5120x5120x8192 (BLAS, %d threads, %.2f s); 1 thread: "
                           "quantise %.2f s, GEMM estimated as the BLAS time x its threads"
                           % (qthreads, t1 - t0, blas_threads, t2 - t1, tq1))
    if workload in ("act_8192x5120", "weight_5120x20480", "tiny_256"):
        # the whole workload (the same tensor the GPU quantises)
        if workload == "act_8192x5120":
            bits, specs = syn.act_8192x5120(), ["row", "col"]
            nbytes = qbytes(8192, 5120, 2)
        elif workload == "weight_5120x20480":
            bits, specs = syn.weight_5120x20480(), ["2d", "2d_t"]
            nbytes = 2 * bits.size + 2 * (bits.size // 2 + bits.size // 256)
        else:
            bits, specs = syn.tiny_256(), ["row"]
            nbytes = qbytes(256, 256)
        t0 = time.perf_counter()
        for s in specs:
            oracle.quantize(bits, s)
        dt = time.perf_counter() - t0
        dt1 = one_thread(lambda: [oracle.quantize(bits, s) for s in specs])
        return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=qthreads, kind="oracle",
                    value_1thread=nbytes / dt1 / 1e9,
                    sample="%s quantise of the whole %dx%d tensor (C oracle, %d threads, %.2f s; 1 thread %.2f s)" % (
                        "+".join(specs), bits.shape[0], bits.shape[1], qthreads, dt, dt1))
    # linear step: one Wgrad GEMM + its two quantisations on a 1/8 token slice
    tokens, hidden, ffn = 2048, 5120, 2560
    dy = syn.laplace(tokens, hidden, 504, 1e-3)
    h = syn.normal(tokens, ffn, 501)
    def run():
        qa = oracle.quantize(dy, "col", "sr", True, 1235, 4321)
        qb = oracle.quantize(h, "col", "rtn", True, 0, 4321)
        oracle.gemm_f64(qa, qb)

    t0 = time.perf_counter()
    run()
    dt = time.perf_counter() - t0
    dt1 = one_thread(run)
    flops = 2.0 * hidden * ffn * tokens
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=max(qthreads, blas_threads), kind="oracle",
                value_1thread=flops / dt1 / 1e12,
                sample="dW2 slice: 2048 tokens, 5120x2560 Wgrad with both column quantisations (%.2f s; "
                       "1 thread %.2f s)" % (dt, dt1))


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wgrad_8192x5120", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-library-gemm", action="store_true",
                    help="skip timing torch.matmul in bf16 on the dominant GEMM's shape")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run steps back to back for this long before the counted warm-up (clock ramp)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps after the timed region with a 512 MiB write before each (caches flushed)")
    ap.add_argument("--breakdown-steps", type=int, default=20,
                    help="steps (at least 1) after the timed region with every call bracketed by events (per-call times)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="run a plain device copy of N MiB (for scaling the HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_bit_quantization_amd as nv
    from nvfp4_bit_quantization_amd import synthetic as syn

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes per copy" % n)
        return
    nv.lib()
    log("setting up", args.workload)
    step, info = WORKLOADS[args.workload](nv, syn)
    torch.cuda.synchronize()

    # Settle: the GPU leaves its idle clock state only after some
    # milliseconds of work, so a short run would time the ramp rather than
    # the kernels (measured: 5 + 20 steps of the Wgrad step gave the GEMM
    # 398-400 us per call where 10 + 100 steps on the same GPU gave 360 us).
    # Steps run back to back for --settle-ms before the counted warm-up
    # steps; nothing about them is timed or reported.
    settle = Timer(live=set())
    n_settle, t_set = 0, time.perf_counter()
    while (time.perf_counter() - t_set) * 1e3 < args.settle_ms:
        for _ in range(4):
            step(settle)
        n_settle += 4
        torch.cuda.synchronize()
    warm = Timer()
    for _ in range(args.warmup):
        step(warm)
    torch.cuda.synchronize()
    log("settle %d steps, warmup done (%d steps)" % (n_settle, args.warmup))

    # timed region: only the dominant call is bracketed by events (its
    # roofline time); the step's wall time gives `value`
    dom = info["dominant"]
    t = Timer(live={dom})
    torch.cuda.synchronize()
    with GpuSampler() as sampler:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(t)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    log("timed %d steps: %.3f ms/step" % (args.steps, ms_step))

    # per-call breakdown, after the timed region: every call bracketed
    tb = Timer()
    for _ in range(max(1, args.breakdown_steps)):
        step(tb)
    torch.cuda.synchronize()

    # cold variant: a 512 MiB write before every step evicts L2 and the
    # 256 MB MALL, so each call starts with its inputs in HBM only
    tc = Timer()
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        for k in range(args.cold_steps):
            flush.fill_(k & 0xFF)
            step(tc)
        torch.cuda.synchronize()
        del flush

    def call_ms(name):
        return t.ms(name) if name == dom else tb.ms(name)

    def rate(c, ms):
        if c["kind"] == "gemm":
            tf = c["flops"] / (ms * 1e-3) / 1e12
            return dict(tflops=round(tf, 1), frac_mfma=round(tf / c.get("peak", MFMA_F16_PEAK_TFLOPS), 4))
        gbs = c["bytes"] / (ms * 1e-3) / 1e9
        return dict(gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))

    parts, cold = {}, {}
    for name, c in info["calls"].items():
        st = t.stats(name) if name == dom else tb.stats(name)
        parts[name] = dict(st, **rate(c, st["ms"]))
        if args.cold_steps > 0:
            cs = tc.stats(name)
            cold[name] = dict(ms_median=cs["ms_median"], ms_min=cs["ms_min"], **rate(c, cs["ms_median"]))

    dc = info["calls"][dom]
    dms = t.ms(dom)
    if dc["kind"] == "gemm":
        achieved = dc["flops"] / (dms * 1e-3) / 1e12
        peak = dc.get("peak", MFMA_F16_PEAK_TFLOPS)
        src = source_hash(*info.get("sources", ("gemm.hip", "gemm_device.hpp", "nvfp4_device.hpp",
                                                "nvfp4_kernels.hpp")))
        traffic = read_traffic("gemm_" + args.workload, src)
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=traffic,
                    kernel=info.get("kernel", "gemm_fast_kernel<4,4>"), ms=round(dms, 4),
                    ms_median=parts[dom]["ms_median"], ms_min=parts[dom]["ms_min"],
                    frac_at_median=round(dc["flops"] / (parts[dom]["ms_median"] * 1e-3) / 1e12 / peak, 4),
                    source_hash=src)
    else:
        achieved = dc["bytes"] / (dms * 1e-3) / 1e9
        src = source_hash("quantize.hip", "quantize_device.hpp", "nvfp4_device.hpp", "nvfp4_kernels.hpp")
        traffic = read_traffic("quantize_" + args.workload, src)
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, kernel="amax+quantize pass",
                    ms=round(dms, 4), ms_median=parts[dom]["ms_median"], ms_min=parts[dom]["ms_min"],
                    source_hash=src)

    if info["flops"] > 0:
        value = info["flops"] / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        value = sum(c["bytes"] for c in info["calls"].values() if c["kind"] == "quantize") / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
    qcalls = [n for n, c in info["calls"].items() if c["kind"] == "quantize"]
    quant = None
    if qcalls:
        qb = sum(info["calls"][n]["bytes"] for n in qcalls)
        qms = sum(call_ms(n) for n in qcalls)
        quant = dict(gbs=round(qb / (qms * 1e-3) / 1e9, 1), frac_hbm=round(qb / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     bytes=qb, ms=round(qms, 4))

    # context for the GEMM roofline: the library's dense bf16 GEMM (torch.matmul,
    # hipBLASLt) on random operands of the dominant GEMM's shape, after the timed
    # region; the NVFP4 GEMM expands 4-bit operands to fp16 and runs at the same
    # MFMA rate, so this is the practical ceiling on this GPU's clocks
    lib_gemm = None
    if dc["kind"] == "gemm" and "M" in dc and not args.no_library_gemm:
        lib_gemm = library_gemm(dc["M"], dc["N"], dc["K"])

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a sample)")
        cpu = cpu_baseline(args.workload, syn)

    out = {
        "metric": "NVFP4 quantize GB/s (% HBM peak); NVFP4 Wgrad GEMM TFLOP/s (% MFMA peak)",
        "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": info.get("dtype", "nvfp4 operands; fp32 quantise math; fp16 MFMA, fp32 accumulate"),
        "data": "synthetic",
        "config": info["config"], "quantize": quant, "calls": parts, "roofline": roof, "cpu_baseline": cpu,
        "cold": cold or None, "gpu_power": sampler.summary(), "settle_steps": n_settle,
    }
    if lib_gemm is not None:
        out["library_bf16_gemm"] = lib_gemm
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
