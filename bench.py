#!/usr/bin/env python3
"""Benchmark of the W8A16 hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
quantize the fp32 weight (per-row bound, fp16 scale, int8 codes; one HIP
kernel) and run the W8A16 matmul with the activations (one HIP kernel).
The default workload is the ChatGLM2-6B-like decode GEMV (M=1, K=4096,
N=27392).  Inputs are seeded synthetic tensors already resident in HBM when
the timed region starts; the step rotates over enough copies of its
operands that the 256 MB Infinity Cache cannot serve them from one step to
the next.

Printed: ONE JSON line with the whole-step throughput (algorithmic bytes of
both kernels / step time, in TB/s), a roofline entry for the kernel that
takes most of the step (its algorithmic bytes / its average duration,
measured with HIP events on the launch stream), per-kernel figures, cold
GEMM-only figures for every workload (decode TB/s, prefill TFLOP/s), cold
figures of the W8A8 (int8 x int8) GEMM with per-token activation
quantization, and the CPU oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
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


def gemm_kernel_name(m, n, k):
    import int8_weight_quantized_amd as qw
    return qw.auto_path(m, n, k)


def rotation_count(bytes_per_set, minimum=2, cap=64):
    return int(min(cap, max(minimum, math.ceil(2 * MALL_BYTES / bytes_per_set))))


class StepRunner:
    """Device buffers for R rotating operand sets of one workload."""

    def __init__(self, wl, sets, with_weights=True):
        import numpy as np
        import torch

        import int8_weight_quantized_amd as qw
        import synthetic
        self.qw, self.torch, self.wl = qw, torch, wl
        x, w = synthetic.make_inputs(wl)
        dev = "cuda:0"
        xd = torch.from_numpy(x).to(dev)
        self.x = [xd] + [xd.clone() for _ in range(sets - 1)]
        if with_weights:
            wd = torch.from_numpy(w).to(dev)
            self.w = [wd] + [wd.clone() for _ in range(sets - 1)]
        else:
            self.w = None
        self.q = [torch.empty((wl.n, wl.k), dtype=torch.int8, device=dev) for _ in range(sets)]
        self.s = [torch.empty((wl.n,), dtype=torch.float16, device=dev) for _ in range(sets)]
        self.y = [torch.empty((wl.m, wl.n), dtype=torch.float16, device=dev) for _ in range(sets)]
        if not with_weights:
            # codes/scales are produced once by the library's own quantizer
            wd = torch.from_numpy(w).to(dev)
            q0, s0 = qw.quantize_weights(wd, wl.clip_percentile)
            for i in range(sets):
                self.q[i].copy_(q0)
                self.s[i].copy_(s0)
            del wd, q0, s0
        del np
        self.sets = sets
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


class W8A8Runner:
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


def time_w8a8(wl, launches=40, warmup=10):
    """Cold W8A8 figures for one workload: the GEMM alone (as
    time_gemm_only) and per-token activation quantization followed by the
    GEMM, each launch pair timed with events."""
    import torch
    r = W8A8Runner(wl, rotation_count(w8a8_bytes(wl.m, wl.n, wl.k) + act_quant_bytes(wl.m, wl.k)))
    avg_ms, med_ms = time_gemm_only(r, launches, warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    torch.cuda.synchronize()
    torch.cuda._sleep(40_000_000)
    for it in range(launches):
        i = it % r.sets
        ev[it][0].record()
        r.quantize(i)
        ev[it][1].record()
        r.gemm(i)
        ev[it][2].record()
    torch.cuda.synchronize()
    aq_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / launches
    pair_ms = sum(e[0].elapsed_time(e[2]) for e in ev) / launches
    ops = gemm_flops(wl.m, wl.n, wl.k)
    mfma = r.qw.w8a8_auto_path(wl.m, wl.n, wl.k) == "mfma"
    tile = list(r.qw.w8a8_tile(wl.m, wl.n, wl.k)) if mfma else None
    sets = r.sets
    del r
    torch.cuda.empty_cache()
    return {"workload": wl.name, "kernel": "w8a8_mfma" if mfma else "w8a8_skinny", "mfma_tile": tile,
            "cold_sets": sets,
            "avg_us": avg_ms * 1e3, "median_us": med_ms * 1e3,
            "TOPs": ops / (avg_ms * 1e-3) / 1e12,
            "mfma_i8_frac": ops / (avg_ms * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS,
            "TBps": w8a8_bytes(wl.m, wl.n, wl.k) / (avg_ms * 1e-3) / 1e12,
            "act_quantize_us": aq_ms * 1e3,
            "act_quantize_plus_gemm_us": pair_ms * 1e3}


class OutlierRunner:
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


def time_outliers(wl, launches=40, warmup=10):
    """Cold figures of the outlier-aware GEMM (dense int8 part plus exact side
    lists) on one workload."""
    import torch
    r = OutlierRunner(wl, rotation_count(gemm_bytes(wl.m, wl.n, wl.k)))
    avg_ms, med_ms = time_gemm_only(r, launches, warmup)
    fl = gemm_flops(wl.m, wl.n, wl.k)
    out = {"workload": wl.name, "kernel": gemm_kernel_name(wl.m, wl.n, wl.k) + "+outliers",
           "slots_per_row": r.cap, "cold_sets": r.sets, "avg_us": avg_ms * 1e3, "median_us": med_ms * 1e3,
           "TFLOPs": fl / (avg_ms * 1e-3) / 1e12,
           "mfma_frac": fl / (avg_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS}
    del r
    torch.cuda.empty_cache()
    return out


def time_full_steps(runner, steps, warmup):
    """Warm up, then time exactly `steps` steps bracketed by synchronizations;
    HIP events on the launch stream time each kernel inside the region."""
    torch = runner.torch
    for it in range(warmup):
        runner.quantize(it % runner.sets)
        runner.gemm(it % runner.sets)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for it in range(steps):
        i = (warmup + it) % runner.sets
        e = ev[it]
        e[0].record()
        runner.quantize(i)
        e[1].record()
        runner.gemm(i)
        e[2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    quant_ms = [e[0].elapsed_time(e[1]) for e in ev]
    gemm_ms = [e[1].elapsed_time(e[2]) for e in ev]
    return (t1 - t0) * 1e3 / steps, sum(quant_ms) / steps, sum(gemm_ms) / steps


def time_gemm_only(runner, launches, warmup):
    """Cold GEMM launches rotating over the operand sets; event pairs per launch.
    A GPU-side sleep is queued first so that every launch is enqueued before
    the GPU reaches it: the event pairs then see device time only, not gaps
    left by host-side launch latency."""
    torch = runner.torch
    for it in range(warmup):
        runner.gemm(it % runner.sets)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    torch.cuda.synchronize()
    torch.cuda._sleep(40_000_000)
    for it in range(launches):
        ev[it][0].record()
        runner.gemm((warmup + it) % runner.sets)
        ev[it][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return sum(ms) / len(ms), ms[len(ms) // 2]


def cpu_baseline(wl, target_s=10.0, max_s=30.0):
    """The oracle as it stands, on the host cores, repeated over full steps of
    the same workload until about `target_s` seconds of work."""
    import oracle
    import synthetic
    x, w = synthetic.make_inputs(wl)
    o = oracle.default()
    steps = 0
    t0 = time.perf_counter()
    while True:
        q, s, _ = o.quantize(w, wl.clip_percentile)
        o.gemm(x, q, s)
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s or el * (steps + 1) / steps > max_s:
            break
    per_step = el / steps
    tbps = (quant_bytes(wl.n, wl.k) + gemm_bytes(wl.m, wl.n, wl.k)) / per_step / 1e12
    return {"value": tbps, "unit": "TB/s", "cores": o.num_threads(), "kind": "oracle",
            "sample": "%d full step(s) of %s (quantize + binary64 GEMM), %.1f s total, %.3f s/step"
                      % (steps, wl.name, el, per_step)}


def sweep_paths(ms=(1, 2, 3, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 512),
                shapes=((4096, 27392), (4096, 4608), (1024, 4096))):
    """Cold timing of each W8A16 and W8A8 GEMM kernel across m (random codes;
    timing only)."""
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
            # kernels this shape supports (a forced kernel outside its limits is refused)
            runs = [(name, launcher(name, path)) for name, path in kernels]
            runs = [(name, f) for name, f in runs if f(0) == 0]
            for it in range(5):
                for j, (_, f) in enumerate(runs):
                    f((it * len(runs) + j) % sets)
            # round-robin: one launch of each kernel per round, so that clock
            # and cache state after the allocations hit every kernel alike
            ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                         for _ in range(30)] for name, _ in runs}
            torch.cuda.synchronize()
            # (every launch takes the next operand set, so none finds its
            # operands in cache)
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="chatglm2_decode_m1_k4096_n27392")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the cold GEMM-only figures")
    ap.add_argument("--only-step", action="store_true", help="time the full steps only (for profiling)")
    ap.add_argument("--sweep-paths", action="store_true",
                    help="only time every GEMM kernel over a range of m (decode -> prefill "
                         "crossover), one JSON line per (shape, m, kernel)")
    ap.add_argument("--only-w8a8", action="store_true",
                    help="only the W8A8 figures of --workload (per-token activation quantization + "
                         "W8A8 GEMM, --steps launches after --warmup), one JSON line (for profiling)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (fp16 negate, 5 launches) so "
                         "that HBM counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the W8A16 path here has no multi-GPU "
              "execution (each GPU would hold its own slice of the weight rows); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

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

    import int8_weight_quantized_amd as qw
    wl = synthetic.BY_NAME[args.workload]
    if args.only_w8a8:
        print(json.dumps(time_w8a8(wl, launches=args.steps, warmup=args.warmup)), flush=True)
        return
    per_set = quant_bytes(wl.n, wl.k) + gemm_bytes(wl.m, wl.n, wl.k)
    sets = rotation_count(per_set)
    runner = StepRunner(wl, sets, with_weights=True)
    ms_step, q_ms, g_ms = time_full_steps(runner, args.steps, args.warmup)

    qb, gb = quant_bytes(wl.n, wl.k), gemm_bytes(wl.m, wl.n, wl.k)
    gname = gemm_kernel_name(wl.m, wl.n, wl.k)
    value = (qb + gb) / (ms_step * 1e-3) / 1e12
    kernels = {
        "quantize": {"avg_us": q_ms * 1e3, "algorithmic_bytes": qb,
                     "achieved_GBps": qb / (q_ms * 1e-3) / 1e9},
        gname: {"avg_us": g_ms * 1e3, "algorithmic_bytes": gb,
                "achieved_GBps": gb / (g_ms * 1e-3) / 1e9,
                "achieved_TFLOPs": gemm_flops(wl.m, wl.n, wl.k) / (g_ms * 1e-3) / 1e12},
    }
    for name, kd in kernels.items():
        kd["hbm_frac"] = kd["achieved_GBps"] / HBM_PEAK_GBPS
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"])
    dk = kernels[dom]
    traffic = measured_traffic(dom, wl.name)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": dk["achieved_GBps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": dk["achieved_GBps"] / HBM_PEAK_GBPS, "traffic": traffic,
                "algorithmic_bytes_per_launch": dk["algorithmic_bytes"], "avg_launch_us": dk["avg_us"]}
    del runner
    torch.cuda.empty_cache()

    secondary = []
    if not args.no_secondary and not args.only_step:
        for other in synthetic.WORKLOADS:
            gbytes = gemm_bytes(other.m, other.n, other.k)
            r = StepRunner(other, rotation_count(gbytes), with_weights=False)
            avg_ms, med_ms = time_gemm_only(r, launches=40, warmup=10)
            fl = gemm_flops(other.m, other.n, other.k)
            kname = gemm_kernel_name(other.m, other.n, other.k)
            ent = {"workload": other.name, "kernel": kname, "cold_sets": r.sets,
                   "mfma_tile": list(qw.mfma_tile(other.m, other.n, other.k)) if kname == "mfma" else None,
                   "avg_us": avg_ms * 1e3, "median_us": med_ms * 1e3,
                   "TBps": gbytes / (avg_ms * 1e-3) / 1e12,
                   "hbm_frac": gbytes / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                   "TFLOPs": fl / (avg_ms * 1e-3) / 1e12,
                   "mfma_frac": fl / (avg_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS}
            secondary.append(ent)
            del r
            torch.cuda.empty_cache()

    w8a8 = []
    if not args.no_secondary and not args.only_step:
        for name in ("small_batch_m8_k4096_n4608", "chatglm2_prefill_m512_k4096_n27392",
                     "transformer_big_ffn_outliers_m4096_k1024_n4096"):
            w8a8.append(time_w8a8(synthetic.BY_NAME[name]))

    tuned = []
    if not args.no_secondary and not args.only_step:
        # per-shape autotuning: time every kernel and tile once, then the
        # automatic call with the record (cold, as gemm_cold)
        for name in ("small_batch_m8_k4096_n4608", "chatglm2_prefill_m512_k4096_n27392",
                     "transformer_big_ffn_outliers_m4096_k1024_n4096"):
            other = synthetic.BY_NAME[name]
            gbytes = gemm_bytes(other.m, other.n, other.k)
            r = StepRunner(other, rotation_count(gbytes), with_weights=False)
            st = qw.w8a16_gemm_tune_raw(r.x[0].data_ptr(), r.q[0].data_ptr(), r.s[0].data_ptr(), r.y[0].data_ptr(),
                                        other.m, other.n, other.k, r.stream)
            if st:
                raise RuntimeError(qw.status_string(st))
            avg_ms, med_ms = time_gemm_only(r, launches=40, warmup=10)
            fl = gemm_flops(other.m, other.n, other.k)
            tuned.append({"workload": name, "choice": qw.tuned_choice(other.m, other.n, other.k),
                          "avg_us": avg_ms * 1e3, "median_us": med_ms * 1e3,
                          "TBps": gbytes / (avg_ms * 1e-3) / 1e12, "TFLOPs": fl / (avg_ms * 1e-3) / 1e12})
            del r
            torch.cuda.empty_cache()
        qw.tune_reset()

    outl = []
    if not args.no_secondary and not args.only_step:
        outl.append(time_outliers(synthetic.BY_NAME["transformer_big_ffn_outliers_m4096_k1024_n4096"]))

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "m": wl.m, "n": wl.n, "k": wl.k,
                   "clip_percentile": wl.clip_percentile, "step": "quantize + w8a16_gemm",
                   "rotation_sets": sets, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "kernels": kernels,
        "gemm_cold": secondary,
        "w8a8_cold": w8a8,
        "outliers_cold": outl,
        "gemm_tuned": tuned,
    }
    if not args.no_cpu_baseline and not args.only_step:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
