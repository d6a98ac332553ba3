"""Sanitizer runs of the host-side C code, on the CPU:

* the oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
  (liboracle_san.so), with every oracle pin run against it in a child process that
  preloads the ASan runtime (leak checking off: the Python interpreter's own allocations
  are not the oracle's);
* the C ABI's host layer (argument validation, size queries, code descriptors) built
  host-only with both sanitizers and linked with stand-ins for the kernel launches, then
  driven through every rejection path and one accepted call per entry point
  (tests/native/abi_validation_check.cpp).
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime not installed")
def test_oracle_pins_under_asan_ubsan():
    env = dict(os.environ)
    env["QTCQ_ORACLE_SANITIZE"] = "1"
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    tests = sorted(os.path.join(HERE, f) for f in os.listdir(HERE)
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + tests, cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=1200)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
    assert os.path.exists(os.path.join(ROOT, "oracle", "liboracle_san.so"))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_layer_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_validation_check"
    cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17",
           "-ffp-contract=off",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "trellis_coded_weight_amd", "csrc"), "-o", str(exe),
           os.path.join(ROOT, "trellis_coded_weight_amd", "csrc", "qtcq.hip"),
           os.path.join(HERE, "native", "abi_validation_check.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
