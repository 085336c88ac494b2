"""Host-side logic of bench.py (CPU only): the algorithmic byte and flop
counts behind the roofline figures, the source hash that ties committed HBM
counters to the code they were measured on, and the one-GPU refusal."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_counts_on_the_decode_workload():
    n, k = 27392, 4096
    # quantizer: fp32 W read once, int8 codes and fp16 scales written
    assert bench.quant_bytes(n, k) == 4 * n * k + n * k + 2 * n == 561042944
    # W8A16 GEMM at M = 1: codes + scales + X read, Y written
    assert bench.gemm_bytes(1, n, k) == n * k + 2 * n + 2 * k + 2 * n == 112315392
    assert bench.gemm_flops(512, n, k) == 2 * 512 * n * k
    # W8A8: int8 activation codes and their fp16 scales instead of fp16 X
    assert bench.w8a8_bytes(8, 4608, 4096) == 4608 * 4096 + 2 * 4608 + 8 * 4096 + 2 * 8 + 2 * 8 * 4608
    assert bench.act_quant_bytes(8, 4096) == 2 * 8 * 4096 + 8 * 4096 + 2 * 8


def _write(d, name, text):
    with open(os.path.join(d, name), "w", encoding="utf-8") as f:
        f.write(text)


def test_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    d = str(tmp_path)
    monkeypatch.setattr(bench, "CSRC", d)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": ["a.hip", "b.h"]})
    _write(d, "a.hip", "int f(int x) {\n    return x + 1; // add one\n}\n")
    _write(d, "b.h", "/* header */\n#define N 4\n")
    h0 = bench.kernel_source_sha("k")
    _write(d, "a.hip", "// a new comment\nint f(int x)\n{\n  return x + 1;  /* still add one */\n}\n")
    assert bench.kernel_source_sha("k") == h0
    _write(d, "a.hip", "int f(int x) {\n    return x + 2; // add one\n}\n")
    assert bench.kernel_source_sha("k") != h0


def test_measured_traffic_is_null_once_the_code_changed(tmp_path, monkeypatch):
    d = str(tmp_path)
    monkeypatch.setattr(bench, "CSRC", d)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"quantize": ["q.hip"]})
    _write(d, "q.hip", "kernel body v1\n")
    tf = os.path.join(d, "traffic.json")
    with open(tf, "w") as f:
        json.dump({"entries": {"wl": {"quantize": {"source_sha": bench.kernel_source_sha("quantize"),
                                                   "hbm_bytes_per_launch": 1234}}}}, f)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", tf)
    assert bench.measured_traffic("quantize", "wl") == 1234
    assert bench.measured_traffic("quantize", "other") is None
    _write(d, "q.hip", "kernel body v2\n")
    assert bench.measured_traffic("quantize", "wl") is None


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
