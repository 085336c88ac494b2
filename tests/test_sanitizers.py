"""Host-side sanitizer runs (CPU only).

Two variant builds are made in a temporary directory and exercised by the
CPU tests in a child process:

* the oracle (plain C) built by gcc with AddressSanitizer and
  UndefinedBehaviorSanitizer, no recovery: the oracle pins run against it;
* libqw with the same sanitizers on its host code only (argument checks,
  kernel choice, the host side of every entry point); GPU code is built
  as usual: the boundary and binding tests run against it (every call
  there is rejected on the host, or fails to launch for want of a GPU).

A sanitizer report fails the child process, and the test with it."""

import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run_child(tests, env_extra, tmp):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow", "-s", "-p", "no:cacheprovider",
           *tests]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_address_and_ub_sanitizers():
    import oracle
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.build(output=os.path.join(tmp, "liboracle_san.so"), extra_flags=SAN)
        libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
        libubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                                  text=True).stdout.strip()
        _run_child(["tests/test_oracle_pins.py"],
                   {"QW_ORACLE_LIBRARY": lib, "LD_PRELOAD": "%s %s" % (libasan, libubsan)}, tmp)


def _clang_asan_runtime():
    llvm = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(llvm):
        return None
    for ver in sorted(os.listdir(llvm), reverse=True):
        p = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_library_host_code_under_address_and_ub_sanitizers():
    rt = _clang_asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc / clang sanitizer runtime")
    from int8_weight_quantized_amd import build as qwbuild
    # each sanitizer flag applies to the host compilation only
    host_only = [f for flag in SAN for f in ("-Xarch_host", flag)]
    with tempfile.TemporaryDirectory() as tmp:
        lib = qwbuild.build(extra=host_only, build_dir=os.path.join(tmp, "obj"),
                            output=os.path.join(tmp, "libqw_san.so"))
        _run_child(["tests/test_boundary.py", "tests/test_binding_validation.py"],
                   {"QW_LIBRARY": lib, "LD_PRELOAD": rt}, tmp)
