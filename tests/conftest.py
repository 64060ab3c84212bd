import os
import sys

# small fp64 matrices dominate the CPU suite; a few BLAS threads avoid oversubscription
os.environ.setdefault("OPENBLAS_NUM_THREADS", "4")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # GPU tests are never skipped silently: without a GPU they fail, so run
    # them with -m gpu on an MI355X and deselect them with -m "not gpu" elsewhere.
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
