import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# The oracle's per-row products are small: one BLAS thread avoids oversubscribing the
# host cores (torch and NumPy would each start a pool per process).
try:
    from threadpoolctl import threadpool_limits
    _LIMITS = threadpool_limits(limits=1)
except Exception:  # threadpoolctl missing: keep the defaults
    _LIMITS = None
