"""Build the gfx950 HIP library libqtcq.so in-tree with hipcc.

Flags that matter for results:
  -ffp-contract=off       the path cost is a chain of separately rounded sub, square,
                          [weight-multiply] and add operations (no fused multiply-add);
  -Xclang -target-feature -Xclang -packed-fp32-ops
                          no packed fp32 instructions (v_pk_*_f32);
  no fast-math / denormal flushing.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "qtcq.hip")
OUT = os.path.join(HERE, "libqtcq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
]


def build_native(verbose: bool = False) -> str:
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_native(verbose=True))
