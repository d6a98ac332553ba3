import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _ensure_native_library():
    # The tests load the in-tree build of the HIP library; only when none exists (a fresh
    # checkout) is it compiled here (hipcc cross-compiles for gfx950 without a GPU).
    lib = os.path.join(ROOT, "trellis_coded_weight_amd", "libqtcq.so")
    if not os.path.exists(lib):
        from trellis_coded_weight_amd import build
        build.build_native()


_ensure_native_library()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
