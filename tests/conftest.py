import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # Load what is built; build only what is missing (a fresh checkout).
    from fp32_gemm_07_amd import build as hip_build
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build(force=True)
    if not os.path.exists(hip_build.LIB_PATH):
        hip_build.build()
