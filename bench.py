#!/usr/bin/env python3
"""Benchmark of the W8A16 GEMM on one MI355X.

The metric is the W8A16 GEMM's effective HBM throughput at decode (M = 1,
the ChatGLM2-6B-like MatMul K = 4096, N = 27392) with its TFLOP/s at
prefill (M = 512) beside it.  One step is one W8A16 GEMM call over one
batch of synthetic input (int8 codes, fp16 scales and activations resident
in HBM); the weight quantizer runs once per weight, offline, so it is timed
separately ("full_step" = quantize + GEMM).  Every timed loop rotates over
enough operand sets (more than twice the 256 MB Infinity Cache) that no
launch finds its weights in cache, and is timed with HIP events on the
launch stream around the whole loop of back-to-back launches: the average
is the sustained per-launch time, which is also what a rocprofv3 kernel
trace of the same loop reports (back-to-back launches leave no gap).

Printed: ONE JSON line with
  value / roofline       decode GEMV: effective TB/s, fraction of 8 TB/s,
                         rocprofv3-counted HBM traffic when measured on the
                         current source;
  roofline_prefill       prefill MFMA GEMM: TFLOP/s, fraction of 2.5 PF;
  stream_ceiling         a plain streaming read of the same bytes;
  sclk_mhz               shader clock right after each timed loop;
  full_step              quantize + GEMM on the decode workload;
  gemm_cold              every workload, GEMM only;
  w8a8_cold, outliers_cold, gemm_tuned   the widened paths;
  cpu_baseline           the CPU oracle on all host cores and on one.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-secondary]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A16 GEMM effective TB/s (decode M=1) and TFLOP/s (prefill M=512), 1×MI355X"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, AMD published
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, AMD published
MFMA_I8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA, AMD published
MALL_BYTES = 256 << 20           # Infinity Cache
DECODE = "chatglm2_decode_m1_k4096_n27392"
PREFILL = "chatglm2_prefill_m512_k4096_n27392"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "int8_weight_quantized_amd", "csrc")
KERNEL_SOURCES = {
    "quantize": ["quantize.hip", "qw_device.h"],
    "gemv": ["gemv.hip", "qw_device.h"],
    "mfma": ["gemm_mfma.hip", "qw_device.h"],
    "skinny": ["gemm_skinny.hip", "qw_device.h"],
}


def quant_bytes(n, k):
    """Algorithmic bytes of the quantizer: read W fp32, write codes and fp16 scales."""
    return 4 * n * k + n * k + 2 * n


def gemm_bytes(m, n, k):
    """Algorithmic bytes of the GEMM: int8 codes, fp16 scales, fp16 X read, fp16 Y written."""
    return n * k + 2 * n + 2 * m * k + 2 * m * n


def gemm_flops(m, n, k):
    return 2 * m * n * k


def w8a8_bytes(m, n, k):
    """Algorithmic bytes of the W8A8 GEMM: int8 weight and activation codes,
    fp16 scales of both, fp16 Y written."""
    return n * k + 2 * n + m * k + 2 * m + 2 * m * n


def act_quant_bytes(m, k):
    """Algorithmic bytes of per-token activation quantization: read X fp16,
    write codes and fp16 scales."""
    return 2 * m * k + m * k + 2 * m


def kernel_source_sha(kernel):
    """Hash of a kernel's sources with comments and whitespace runs removed,
    so that documentation edits do not void the counters measured on the
    code."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs, or None when absent or when the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
        ent = data["entries"][workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if ent.get("source_sha") != kernel_source_sha(kernel):
        return None
    return ent.get("hbm_bytes_per_launch")


def rotation_count(bytes_per_set, minimum=2, cap=64):
    """Operand sets whose total exceeds twice the Infinity Cache."""
    return int(min(cap, max(minimum, math.ceil(2 * MALL_BYTES / bytes_per_set))))


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

class Clock:
    """The shader clock right after a timed loop (library probe: shader-clock
    ticks against the 100 MHz constant clock over a 20 us spin)."""

    def __init__(self):
        import torch

        import int8_weight_quantized_amd as qw
        self.qw, self.torch = qw, torch
        self.buf = torch.zeros(2, dtype=torch.int64, device="cuda:0")

    def enqueue(self, stream):
        st = self.qw.probe_shader_clock_raw(self.buf.data_ptr(), stream)
        if st:
            raise RuntimeError(self.qw.status_string(st))

    def mhz(self):
        ticks, ref = (int(v) for v in self.buf.cpu().tolist())
        return 100.0 * ticks / ref if ref > 0 else None


def timed_loop(launch, sets, launches, warmup, clock=None, stream=None):
    """Sustained per-launch time (ms) of `launches` back-to-back launches,
    each on the next operand set, after `warmup` untimed ones.  A GPU-side
    sleep is queued first so that every launch is enqueued before the GPU
    reaches the start event: the event pair then brackets device time only.
    Returns (ms per launch, wall ms of the bracket, clock MHz or None)."""
    import torch
    for it in range(warmup):
        launch(it % sets)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(20_000_000)
    a.record()
    for it in range(launches):
        launch((warmup + it) % sets)
    b.record()
    if clock is not None:
        clock.enqueue(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return a.elapsed_time(b) / launches, wall, (clock.mhz() if clock is not None else None)


# ---------------------------------------------------------------------------
# operand sets
# ---------------------------------------------------------------------------

class GemmSets:
    """R rotating W8A16 operand sets of one workload, codes and scales from
    the library's own quantizer (or, with `with_weights`, the fp32 weights
    too, for the quantize + GEMM step)."""

    def __init__(self, wl, sets, with_weights=False):
        import torch

        import int8_weight_quantized_amd as qw
        import synthetic
        self.qw, self.torch, self.wl, self.sets = qw, torch, wl, sets
        x, w = synthetic.make_inputs(wl)
        dev = "cuda:0"
        xd = torch.from_numpy(x).to(dev)
        self.x = [xd] + [xd.clone() for _ in range(sets - 1)]
        wd = torch.from_numpy(w).to(dev)
        del x, w
        self.w = ([wd] + [wd.clone() for _ in range(sets - 1)]) if with_weights else None
        q0, s0 = qw.quantize_weights(wd, wl.clip_percentile)
        self.q = [q0] + [q0.clone() for _ in range(sets - 1)]
        self.s = [s0] + [s0.clone() for _ in range(sets - 1)]
        self.y = [torch.empty((wl.m, wl.n), dtype=torch.float16, device=dev) for _ in range(sets)]
        self.stream = int(torch.cuda.current_stream().cuda_stream)

    def quantize(self, i):
        wl = self.wl
        st = self.qw.quantize_weights_raw(self.w[i].data_ptr(), wl.n, wl.k, wl.clip_percentile,
                                          self.q[i].data_ptr(), self.s[i].data_ptr(), self.stream)
        if st:
            raise RuntimeError(self.qw.status_string(st))

    def gemm(self, i):
        wl = self.wl
        st = self.qw.w8a16_gemm_raw(self.x[i].data_ptr(), self.q[i].data_ptr(), self.s[i].data_ptr(),
                                    self.y[i].data_ptr(), wl.m, wl.n, wl.k, self.stream, 0)
        if st:
            raise RuntimeError(self.qw.status_string(st))


class W8A8Sets:
    """Rotating operand sets for the W8A8 path: fp16 activations quantized
    per token (the library's quantizer), int8 weight codes quantized once."""

    def __init__(self, wl, sets):
        import torch

        import int8_weight_quantized_amd as qw
        import synthetic
        self.qw, self.torch, self.wl, self.sets = qw, torch, wl, sets
        x, w = synthetic.make_inputs(wl)
        dev = "cuda:0"
        xd = torch.from_numpy(x).to(dev)
        self.x = [xd] + [xd.clone() for _ in range(sets - 1)]
        wd = torch.from_numpy(w).to(dev)
        q0, s0 = qw.quantize_weights(wd, wl.clip_percentile)
        del wd
        self.q = [q0] + [q0.clone() for _ in range(sets - 1)]
        self.s = [s0] + [s0.clone() for _ in range(sets - 1)]
        self.qx = [torch.empty((wl.m, wl.k), dtype=torch.int8, device=dev) for _ in range(sets)]
        self.sx = [torch.empty((wl.m,), dtype=torch.float16, device=dev) for _ in range(sets)]
        self.y = [torch.empty((wl.m, wl.n), dtype=torch.float16, device=dev) for _ in range(sets)]
        self.stream = int(torch.cuda.current_stream().cuda_stream)
        for i in range(sets):
            self.quantize(i)

    def quantize(self, i):
        wl = self.wl
        st = self.qw.quantize_weights_f16_raw(self.x[i].data_ptr(), wl.m, wl.k, 100.0, self.qx[i].data_ptr(),
                                              self.sx[i].data_ptr(), self.stream)
        if st:
            raise RuntimeError(self.qw.status_string(st))

    def gemm(self, i):
        wl = self.wl
        st = self.qw.w8a8_gemm_raw(self.qx[i].data_ptr(), self.sx[i].data_ptr(), self.q[i].data_ptr(),
                                   self.s[i].data_ptr(), self.y[i].data_ptr(), wl.m, wl.n, wl.k, self.stream)
        if st:
            raise RuntimeError(self.qw.status_string(st))

    def quantize_and_gemm(self, i):
        self.quantize(i)
        self.gemm(i)


class OutlierSets:
    """Rotating operand sets for the outlier-aware W8A16 GEMM: weights
    quantized once with side lists (the library's quantizer)."""

    def __init__(self, wl, sets):
        import torch

        import int8_weight_quantized_amd as qw
        import synthetic
        self.qw, self.torch, self.wl, self.sets = qw, torch, wl, sets
        x, w = synthetic.make_inputs(wl)
        dev = "cuda:0"
        xd = torch.from_numpy(x).to(dev)
        self.x = [xd] + [xd.clone() for _ in range(sets - 1)]
        wd = torch.from_numpy(w).to(dev)
        q0, s0, i0, v0 = qw.quantize_weights_outliers(wd, wl.clip_percentile)
        del wd
        self.cap = i0.shape[1]
        self.q = [q0] + [q0.clone() for _ in range(sets - 1)]
        self.s = [s0] + [s0.clone() for _ in range(sets - 1)]
        self.i = [i0.contiguous()] + [i0.contiguous().clone() for _ in range(sets - 1)]
        self.v = [v0.contiguous()] + [v0.contiguous().clone() for _ in range(sets - 1)]
        self.y = [torch.empty((wl.m, wl.n), dtype=torch.float16, device=dev) for _ in range(sets)]
        self.stream = int(torch.cuda.current_stream().cuda_stream)

    def gemm(self, i):
        wl = self.wl
        st = self.qw.w8a16_gemm_outliers_raw(self.x[i].data_ptr(), self.q[i].data_ptr(), self.s[i].data_ptr(),
                                             self.i[i].data_ptr(), self.v[i].data_ptr(), self.cap,
                                             self.y[i].data_ptr(), wl.m, wl.n, wl.k, self.stream, 0)
        if st:
            raise RuntimeError(self.qw.status_string(st))


def gemm_entry(wl, avg_ms, wall_ms, mhz, sets, launches, kernel, tile=None):
    gb, fl = gemm_bytes(wl.m, wl.n, wl.k), gemm_flops(wl.m, wl.n, wl.k)
    return {"workload": wl.name, "kernel": kernel, "mfma_tile": tile, "cold_sets": sets, "launches": launches,
            "avg_us": avg_ms * 1e3, "TBps": gb / (avg_ms * 1e-3) / 1e12,
            "hbm_frac": gb / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "TFLOPs": fl / (avg_ms * 1e-3) / 1e12,
            "mfma_frac": fl / (avg_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "sclk_mhz_after": mhz, "loop_wall_ms": wall_ms}


def time_gemm(wl, launches, warmup, clock):
    """Cold GEMM-only figures of one workload (automatic kernel choice)."""
    import torch
    r = GemmSets(wl, rotation_count(gemm_bytes(wl.m, wl.n, wl.k)))
    avg, wall, mhz = timed_loop(r.gemm, r.sets, launches, warmup, clock, r.stream)
    kname = r.qw.auto_path(wl.m, wl.n, wl.k)
    tile = list(r.qw.mfma_tile(wl.m, wl.n, wl.k)) if kname == "mfma" else None
    ent = gemm_entry(wl, avg, wall, mhz, r.sets, launches, kname, tile)
    del r
    torch.cuda.empty_cache()
    return ent


def time_w8a8(wl, launches, warmup, clock):
    """Cold W8A8 figures for one workload: the GEMM alone and per-token
    activation quantization followed by the GEMM."""
    import torch
    r = W8A8Sets(wl, rotation_count(w8a8_bytes(wl.m, wl.n, wl.k) + act_quant_bytes(wl.m, wl.k)))
    avg, wall, mhz = timed_loop(r.gemm, r.sets, launches, warmup, clock, r.stream)
    pair, _, _ = timed_loop(r.quantize_and_gemm, r.sets, launches, warmup)
    ops = gemm_flops(wl.m, wl.n, wl.k)
    mfma = r.qw.w8a8_auto_path(wl.m, wl.n, wl.k) == "mfma"
    tile = list(r.qw.w8a8_tile(wl.m, wl.n, wl.k)) if mfma else None
    sets = r.sets
    del r
    torch.cuda.empty_cache()
    return {"workload": wl.name, "kernel": "w8a8_mfma" if mfma else "w8a8_skinny", "mfma_tile": tile,
            "cold_sets": sets, "launches": launches, "avg_us": avg * 1e3,
            "TOPs": ops / (avg * 1e-3) / 1e12,
            "mfma_i8_frac": ops / (avg * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS,
            "TBps": w8a8_bytes(wl.m, wl.n, wl.k) / (avg * 1e-3) / 1e12,
            "act_quantize_plus_gemm_us": pair * 1e3, "sclk_mhz_after": mhz}


def time_outliers(wl, launches, warmup, clock):
    """Cold figures of the outlier-aware GEMM (dense int8 part plus exact side
    lists) on one workload."""
    import torch
    r = OutlierSets(wl, rotation_count(gemm_bytes(wl.m, wl.n, wl.k)))
    avg, wall, mhz = timed_loop(r.gemm, r.sets, launches, warmup, clock, r.stream)
    fl = gemm_flops(wl.m, wl.n, wl.k)
    out = {"workload": wl.name, "kernel": r.qw.auto_path(wl.m, wl.n, wl.k) + "+outliers",
           "slots_per_row": r.cap, "cold_sets": r.sets, "launches": launches, "avg_us": avg * 1e3,
           "TFLOPs": fl / (avg * 1e-3) / 1e12,
           "mfma_frac": fl / (avg * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, "sclk_mhz_after": mhz}
    del r
    torch.cuda.empty_cache()
    return out


def time_tuned(wl, launches, warmup, clock):
    """Per-shape autotuning: time every kernel and tile once on the first
    operand set, then the automatic call with the record (cold)."""
    import torch
    r = GemmSets(wl, rotation_count(gemm_bytes(wl.m, wl.n, wl.k)))
    st = r.qw.w8a16_gemm_tune_raw(r.x[0].data_ptr(), r.q[0].data_ptr(), r.s[0].data_ptr(), r.y[0].data_ptr(),
                                  wl.m, wl.n, wl.k, r.stream)
    if st:
        raise RuntimeError(r.qw.status_string(st))
    avg, wall, mhz = timed_loop(r.gemm, r.sets, launches, warmup, clock, r.stream)
    choice = r.qw.tuned_choice(wl.m, wl.n, wl.k)
    del r
    torch.cuda.empty_cache()
    ent = gemm_entry(wl, avg, wall, mhz, rotation_count(gemm_bytes(wl.m, wl.n, wl.k)), launches, "tuned")
    ent["choice"] = choice
    return ent


def time_full_step(wl, launches, warmup, clock):
    """Quantize + GEMM on one workload, each kernel timed in its own
    back-to-back loop and the pair as a loop of steps."""
    import torch
    sets = rotation_count(quant_bytes(wl.n, wl.k) + gemm_bytes(wl.m, wl.n, wl.k))
    r = GemmSets(wl, sets, with_weights=True)

    def step(i):
        r.quantize(i)
        r.gemm(i)
    q_ms, _, _ = timed_loop(r.quantize, sets, launches, warmup)
    s_ms, _, mhz = timed_loop(step, sets, launches, warmup, clock, r.stream)
    del r
    torch.cuda.empty_cache()
    qb, gb = quant_bytes(wl.n, wl.k), gemm_bytes(wl.m, wl.n, wl.k)
    return {"workload": wl.name, "step": "quantize + w8a16_gemm", "cold_sets": sets, "launches": launches,
            "step_us": s_ms * 1e3, "step_TBps": (qb + gb) / (s_ms * 1e-3) / 1e12,
            "quantize_us": q_ms * 1e3, "quantize_algorithmic_bytes": qb,
            "quantize_TBps": qb / (q_ms * 1e-3) / 1e12, "quantize_hbm_frac": qb / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "sclk_mhz_after": mhz}


def time_stream_ceiling(nbytes, launches, warmup, clock):
    """The plain streaming-read probe over rotating buffers of `nbytes`."""
    import torch

    import int8_weight_quantized_amd as qw
    sets = rotation_count(nbytes)
    bufs = [torch.ones(nbytes, dtype=torch.int8, device="cuda:0") for _ in range(sets)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    stream = int(torch.cuda.current_stream().cuda_stream)

    def launch(i):
        st = qw.probe_stream_read_raw(bufs[i].data_ptr(), nbytes, 0x5eed1234, sink.data_ptr(), stream)
        if st:
            raise RuntimeError(qw.status_string(st))
    avg, wall, mhz = timed_loop(launch, sets, launches, warmup, clock, stream)
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "cold_sets": sets, "launches": launches, "avg_us": avg * 1e3,
            "TBps": nbytes / (avg * 1e-3) / 1e12, "hbm_frac": nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "sclk_mhz_after": mhz}


# ---------------------------------------------------------------------------
# the CPU oracle as a baseline
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or None


def _repeat(fn, min_s):
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return el / n, n


def cpu_leg(threads, min_s):
    """One leg of the CPU baseline, run in a child process whose OpenMP
    thread count is fixed by its environment: the oracle's quantizer and
    binary64 GEMM on (samples of) the decode, prefill and FFN workloads."""
    import oracle
    import synthetic
    o = oracle.default()
    out = {"threads": o.num_threads(), "legs": []}
    dec = synthetic.BY_NAME[DECODE]
    x, w = synthetic.make_inputs(dec)
    q, s, _ = o.quantize(w, dec.clip_percentile)
    sec, reps = _repeat(lambda: o.quantize(w, dec.clip_percentile), min_s)
    out["legs"].append({"what": "quantize", "workload": dec.name, "rows": dec.n, "s": sec, "reps": reps,
                        "GBps": quant_bytes(dec.n, dec.k) / sec / 1e9})
    sec, reps = _repeat(lambda: o.gemm(x, q, s), min_s)
    out["legs"].append({"what": "gemm", "workload": dec.name, "m_rows": dec.m, "s": sec, "reps": reps,
                        "TBps": gemm_bytes(dec.m, dec.n, dec.k) / sec / 1e12,
                        "GFLOPs": gemm_flops(dec.m, dec.n, dec.k) / sec / 1e9})
    pre = synthetic.BY_NAME[PREFILL]
    xp, _ = synthetic.make_inputs(pre)  # same weight as decode (same seed and shape)
    rows = 8 if threads > 1 else 1
    sec, reps = _repeat(lambda: o.gemm(xp[:rows], q, s), min_s)
    out["legs"].append({"what": "gemm", "workload": pre.name, "m_rows": rows, "s": sec, "reps": reps,
                        "GFLOPs": gemm_flops(rows, pre.n, pre.k) / sec / 1e9})
    del x, w, q, s, xp
    ffn = synthetic.BY_NAME["transformer_big_ffn_outliers_m4096_k1024_n4096"]
    x, w = synthetic.make_inputs(ffn)
    q, s, _ = o.quantize(w, ffn.clip_percentile)
    sec, reps = _repeat(lambda: o.quantize(w, ffn.clip_percentile), min_s)
    out["legs"].append({"what": "quantize", "workload": ffn.name, "rows": ffn.n, "s": sec, "reps": reps,
                        "GBps": quant_bytes(ffn.n, ffn.k) / sec / 1e9})
    rows = 32 if threads > 1 else 4
    sec, reps = _repeat(lambda: o.gemm(x[:rows], q, s), min_s)
    out["legs"].append({"what": "gemm", "workload": ffn.name, "m_rows": rows, "s": sec, "reps": reps,
                        "GFLOPs": gemm_flops(rows, ffn.n, ffn.k) / sec / 1e9})
    return out


def cpu_baseline(gpu):
    """The oracle as it stands, timed in child processes on all host cores
    and on one core, each leg repeated for about a second; `gpu` holds the
    GPU figures each leg is compared with."""
    legs = {}
    host = os.cpu_count() or 1
    for threads in (host, 1):
        env = dict(os.environ)
        env.update({"OMP_NUM_THREADS": str(threads), "OMP_PROC_BIND": "close"})
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-leg", str(threads)], env=env,
                             capture_output=True, text=True, timeout=600, cwd=ROOT)
        if res.returncode != 0:
            raise RuntimeError("cpu baseline leg failed:\n" + res.stderr[-2000:])
        legs[threads] = json.loads(res.stdout.strip().splitlines()[-1])
    full = legs[host]
    for leg in full["legs"] + legs[1]["legs"]:
        g = gpu.get((leg["what"], leg["workload"]))
        if g is None:
            continue
        if leg["what"] == "quantize":
            leg["gpu_s"] = g
            leg["gpu_speedup"] = leg["s"] / g
        else:
            # the CPU ran the first m_rows activation rows; scaled to the whole workload
            leg["gpu_s"] = g
            leg["gpu_speedup"] = leg["s"] / leg["m_rows"] * synthetic_rows(leg["workload"]) / g
    dec = next(l for l in full["legs"] if l["what"] == "gemm" and l["workload"] == DECODE)
    return {"value": dec["TBps"], "unit": "TB/s", "cores": full["threads"], "kind": "oracle",
            "sample": "oracle binary64 W8A16 GEMM on the full decode workload (1 x 4096 x 27392), repeated "
                      "for about a second; further legs below: the quantizer on the decode and FFN weights, "
                      "the GEMM on the first rows of the prefill and FFN activations (GFLOP/s scaled by rows), "
                      "each on all host threads and on one",
            "host_cpus": host, "cpu_model": cpu_model(),
            "all_cores": full, "one_core": legs[1]}


def synthetic_rows(name):
    import synthetic
    return synthetic.BY_NAME[name].m


# ---------------------------------------------------------------------------
# other modes
# ---------------------------------------------------------------------------

def sweep_paths(ms=(1, 2, 3, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 512),
                shapes=((4096, 27392), (4096, 4608), (1024, 4096))):
    """Cold timing of each W8A16 and W8A8 GEMM kernel across m (random codes;
    timing only), round-robin over the kernels with a fresh operand set per
    launch."""
    import torch

    import int8_weight_quantized_amd as qw
    stream = int(torch.cuda.current_stream().cuda_stream)
    for (k, n) in shapes:
        for m in ms:
            gbytes = gemm_bytes(m, n, k)
            sets = rotation_count(gbytes)
            g = torch.Generator(device="cuda:0").manual_seed(m)
            q = [torch.randint(-127, 128, (n, k), dtype=torch.int8, device="cuda:0", generator=g)
                 for _ in range(sets)]
            s = [torch.rand((n,), device="cuda:0", generator=g).half() * 1e-3 for _ in range(sets)]
            x = [torch.randn((m, k), device="cuda:0", generator=g).half() for _ in range(sets)]
            qx = [torch.randint(-127, 128, (m, k), dtype=torch.int8, device="cuda:0", generator=g)
                  for _ in range(sets)]
            sx = [torch.rand((m,), device="cuda:0", generator=g).half() * 1e-2 for _ in range(sets)]
            y = [torch.empty((m, n), dtype=torch.float16, device="cuda:0") for _ in range(sets)]
            kernels = (("gemv", 1), ("skinny", 3), ("mfma", 2), ("w8a8_skinny", 3), ("w8a8_mfma", 2))

            def launcher(name, path):
                if name.startswith("w8a8"):
                    return lambda i: qw.w8a8_gemm_raw(qx[i].data_ptr(), sx[i].data_ptr(), q[i].data_ptr(),
                                                      s[i].data_ptr(), y[i].data_ptr(), m, n, k, stream, path)
                return lambda i: qw.w8a16_gemm_raw(x[i].data_ptr(), q[i].data_ptr(), s[i].data_ptr(),
                                                   y[i].data_ptr(), m, n, k, stream, path)
            runs = [(name, launcher(name, path)) for name, path in kernels]
            runs = [(name, f) for name, f in runs if f(0) == 0]
            for it in range(5):
                for j, (_, f) in enumerate(runs):
                    f((it * len(runs) + j) % sets)
            ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                         for _ in range(30)] for name, _ in runs}
            torch.cuda.synchronize()
            for it in range(30):
                for j, (name, f) in enumerate(runs):
                    ev[name][it][0].record()
                    f((it * len(runs) + j) % sets)
                    ev[name][it][1].record()
            torch.cuda.synchronize()
            for name, _ in runs:
                ms_ = sorted(a.elapsed_time(b) for a, b in ev[name])
                avg = sum(ms_) / len(ms_)
                print(json.dumps({"sweep": "gemm_paths", "k": k, "n": n, "m": m, "kernel": name,
                                  "auto": qw.auto_path(m, n, k), "auto_w8a8": qw.w8a8_auto_path(m, n, k),
                                  "avg_us": avg * 1e3,
                                  "median_us": ms_[len(ms_) // 2] * 1e3,
                                  "TBps": (w8a8_bytes(m, n, k) if name.startswith("w8a8") else gbytes)
                                  / (avg * 1e-3) / 1e12,
                                  "TFLOPs": gemm_flops(m, n, k) / (avg * 1e-3) / 1e12}), flush=True)
            del q, s, x, qx, sx, y
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed decode GEMM launches (one step each)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="only the headline decode and prefill figures and the stream ceiling")
    ap.add_argument("--only-gemm", metavar="WORKLOAD",
                    help="only the cold GEMM loop of one workload (--steps launches), one JSON line "
                         "(for rocprofv3 kernel traces and counters)")
    ap.add_argument("--only-step", action="store_true",
                    help="only quantize + GEMM steps of the decode workload (for rocprofv3)")
    ap.add_argument("--only-w8a8", metavar="WORKLOAD",
                    help="only the W8A8 figures of one workload, one JSON line (for rocprofv3)")
    ap.add_argument("--only-stream-ceiling", action="store_true",
                    help="only the plain streaming read of the decode weight's bytes (for rocprofv3)")
    ap.add_argument("--sweep-paths", action="store_true",
                    help="only time every GEMM kernel over a range of m (decode -> prefill crossover), "
                         "one JSON line per (shape, m, kernel)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (fp16 negate, 5 launches) so that HBM "
                         "counters can be scaled against a kernel of known traffic")
    ap.add_argument("--cpu-leg", type=int, default=0, metavar="THREADS", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the W8A16 path here has no multi-GPU "
              "execution (each GPU would hold its own slice of the weight rows); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.cpu_leg:
        print(json.dumps(cpu_leg(args.cpu_leg, 1.0)), flush=True)
        return

    import torch

    import synthetic
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": nbytes, "calibrate_copy_bytes_written": nbytes,
                          "launches": 5}), flush=True)
        return

    if args.sweep_paths:
        sweep_paths()
        return

    clock = Clock()
    if args.only_gemm:
        print(json.dumps(time_gemm(synthetic.BY_NAME[args.only_gemm], args.steps, args.warmup, clock)),
              flush=True)
        return
    if args.only_w8a8:
        print(json.dumps(time_w8a8(synthetic.BY_NAME[args.only_w8a8], args.steps, args.warmup, clock)),
              flush=True)
        return
    if args.only_step:
        print(json.dumps(time_full_step(synthetic.BY_NAME[DECODE], args.steps, args.warmup, clock)), flush=True)
        return
    if args.only_stream_ceiling:
        dec = synthetic.BY_NAME[DECODE]
        print(json.dumps(time_stream_ceiling(dec.n * dec.k, args.steps, args.warmup, clock)), flush=True)
        return

    # ---- headline: the decode GEMV, cold, K back-to-back steps ----
    dec = synthetic.BY_NAME[DECODE]
    head = time_gemm(dec, args.steps, args.warmup, clock)
    print("[bench] decode gemm %.2f us, %.3f TB/s" % (head["avg_us"], head["TBps"]), file=sys.stderr, flush=True)
    gb = gemm_bytes(dec.m, dec.n, dec.k)
    roofline = {"bound": "hbm", "kernel": head["kernel"], "workload": dec.name,
                "achieved": gb / (head["avg_us"] * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": gb / (head["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                "traffic": measured_traffic(head["kernel"], dec.name),
                "algorithmic_bytes_per_launch": gb, "avg_launch_us": head["avg_us"],
                "sclk_mhz_after": head["sclk_mhz_after"]}
    pre = synthetic.BY_NAME[PREFILL]
    pf = time_gemm(pre, 40, 10, clock)
    print("[bench] prefill gemm %.2f us, %.1f TFLOP/s" % (pf["avg_us"], pf["TFLOPs"]), file=sys.stderr, flush=True)
    roofline_prefill = {"bound": "mfma", "kernel": pf["kernel"], "mfma_tile": pf["mfma_tile"], "workload": pre.name,
                        "achieved": pf["TFLOPs"], "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": pf["mfma_frac"], "traffic": measured_traffic(pf["kernel"], pre.name),
                        "algorithmic_flops_per_launch": gemm_flops(pre.m, pre.n, pre.k),
                        "algorithmic_bytes_per_launch": gemm_bytes(pre.m, pre.n, pre.k),
                        "avg_launch_us": pf["avg_us"], "sclk_mhz_after": pf["sclk_mhz_after"]}
    ceiling = time_stream_ceiling(dec.n * dec.k, 40, 10, clock)
    print("[bench] stream ceiling %.2f us" % ceiling["avg_us"], file=sys.stderr, flush=True)

    secondary = {}
    if not args.no_secondary:
        secondary["full_step"] = time_full_step(dec, 40, 10, clock)
        cold = []
        for wl in synthetic.WORKLOADS:
            if wl.name == dec.name:
                cold.append(head)
            elif wl.name == pre.name:
                cold.append(pf)
            else:
                cold.append(time_gemm(wl, 40, 10, clock))
        secondary["gemm_cold"] = cold
        print("[bench] gemm_cold done", file=sys.stderr, flush=True)
        secondary["w8a8_cold"] = [time_w8a8(synthetic.BY_NAME[n], 40, 10, clock)
                                  for n in ("small_batch_m8_k4096_n4608", PREFILL,
                                            "transformer_big_ffn_outliers_m4096_k1024_n4096")]
        secondary["outliers_cold"] = [time_outliers(synthetic.BY_NAME["transformer_big_ffn_outliers_m4096_k1024_n4096"],
                                                    40, 10, clock)]
        import int8_weight_quantized_amd as qw
        secondary["gemm_tuned"] = [time_tuned(synthetic.BY_NAME[n], 40, 10, clock)
                                   for n in ("small_batch_m8_k4096_n4608", PREFILL,
                                             "transformer_big_ffn_outliers_m4096_k1024_n4096")]
        qw.tune_reset()
        print("[bench] secondary done", file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": head["TBps"],
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["avg_us"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": dec.name, "m": dec.m, "n": dec.n, "k": dec.k,
                   "step": "one w8a16_gemm call (int8 codes + fp16 scales + fp16 X -> fp16 Y)",
                   "rotation_sets": head["cold_sets"], "timing": "HIP events around K back-to-back launches",
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "roofline_prefill": roofline_prefill,
        "prefill_TFLOPs": pf["TFLOPs"],
        "stream_ceiling": ceiling,
        "sclk_mhz": {"after_decode_loop": head["sclk_mhz_after"], "after_prefill_loop": pf["sclk_mhz_after"]},
    }
    result.update(secondary)
    if not args.no_cpu_baseline:
        gpu = {("quantize", dec.name): (secondary.get("full_step") or {}).get("quantize_us", 0) * 1e-6 or None,
               ("gemm", dec.name): head["avg_us"] * 1e-6, ("gemm", pre.name): pf["avg_us"] * 1e-6}
        for ent in secondary.get("gemm_cold", []):
            gpu[("gemm", ent["workload"])] = ent["avg_us"] * 1e-6
        gpu = {key: v for key, v in gpu.items() if v}
        result["cpu_baseline"] = cpu_baseline(gpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
