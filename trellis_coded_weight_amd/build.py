"""Build the gfx950 HIP library libqtcq.so in-tree with hipcc.

The library is one C-ABI unit (csrc/qtcq.hip) and one launch unit per kernel family
(csrc/launch_*.hip).  Each is compiled to an object on its own, in parallel, and the
objects are linked into the shared library.

Flags that matter for results:
  -ffp-contract=off       the path cost is a chain of separately rounded sub, square,
                          [weight-multiply] and add operations (no fused multiply-add);
  -Xclang -target-feature -Xclang -packed-fp32-ops
                          no packed fp32 instructions (v_pk_*_f32);
  no fast-math / denormal flushing.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqtcq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def sources() -> list[str]:
    return [os.path.join(CSRC, "qtcq.hip")] + sorted(glob.glob(os.path.join(CSRC, "launch_*.hip")))


def _jobs() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, int(os.environ.get("MAX_JOBS", n)), 16))


def build_native(verbose: bool = False) -> str:
    tmpdir = tempfile.mkdtemp(prefix="qtcq_build_")
    try:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC] + FLAGS + ["-c", "-o", obj, src]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError("hipcc failed on %s:\n%s%s" % (src, res.stdout, res.stderr))
            if verbose:
                print(" ".join(cmd))
            return obj

        # the largest units first, so the slowest compile starts earliest
        srcs = sorted(sources(), key=os.path.getsize, reverse=True)
        with ThreadPoolExecutor(_jobs()) as pool:
            objs = list(pool.map(compile_one, srcs))
        tmp = OUT + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
        if verbose:
            print(" ".join(cmd))
        os.replace(tmp, OUT)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return OUT


if __name__ == "__main__":
    print(build_native(verbose=True))
