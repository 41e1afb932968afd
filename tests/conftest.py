import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only oracle runs")
    if os.environ.get("BCJR_SANITIZE") == "1":
        # the CPU sanitizer run (tests/run_sanitizers.py): the library with sanitized host code
        from bcjr_soft_decoding_amd import bcjr, build

        bcjr.LIB_PATH = build.SAN_LIB
