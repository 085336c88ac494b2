"""Build libqw.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python -m int8_weight_quantized_amd.build [-v]

Each translation unit is compiled with hipcc for gfx950 only, then linked
into ``int8_weight_quantized_amd/libqw.so``.  Flags worth knowing:
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the compiler
    from emitting packed fp32 VALU instructions (harmless host-pass warning);
  * ``-ffp-contract=off`` on the quantizer and the C ABI unit: the rounding
    contract of the quantizer forbids fused multiply-add;
  * no fast-math anywhere; fp32 division stays correctly rounded (hipcc's
    default -fhip-fp32-correctly-rounded-divide-sqrt).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libqw.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
UNITS = {
    "qw_api.hip": ["-ffp-contract=off"],
    "quantize.hip": ["-ffp-contract=off"],
    "gemv.hip": [],
    "gemm_mfma.hip": [],
    "gemm_skinny.hip": [],
    "tune.hip": [],
    "probe.hip": [],
}


def _compile(unit: str, extra, verbose: bool, defines=(), build_dir: str = BUILD_DIR) -> str:
    src = os.path.join(CSRC, unit)
    obj = os.path.join(build_dir, unit.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *extra, *defines, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (unit, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, defines=(), extra=(), build_dir: str = BUILD_DIR, output: str = LIBRARY) -> str:
    """Compile every HIP unit and link libqw.so; returns the library path.

    `extra` adds compiler flags to every unit and `build_dir` / `output`
    place a variant build elsewhere (the host-sanitizer build of the CPU
    tests uses both)."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(UNITS))) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], [*kv[1], *extra], verbose, defines, build_dir),
                           UNITS.items()))
    tmp = output + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(verbose=args.verbose))
