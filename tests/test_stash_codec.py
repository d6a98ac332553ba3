"""The BCJR stash codec and normaliser rounding, checked on the CPU: a small harness
(tests/native/stash_codec_check.hip) includes the kernels' header and calls the same
inline functions on the host.  Built with hipcc's host compilation only."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_stash_codec_on_host(tmp_path):
    exe = tmp_path / "stash_codec_check"
    src = os.path.join(HERE, "native", "stash_codec_check.hip")
    cmd = [HIPCC, "--offload-arch=gfx950", "--cuda-host-only", "-O2", "-std=c++17",
           "-ffp-contract=off", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "trellis_coded_weight_amd", "csrc"), "-o", str(exe), src]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
