import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _ensure_built():
    """Build the HIP library and the oracle only if nothing is built yet (a
    fresh checkout); otherwise use what is there."""
    lib = os.path.join(ROOT, "bit_weight_only_03_amd", "libw4a16.so")
    if not os.path.exists(lib):
        from bit_weight_only_03_amd import build as _b
        _b.build()
    import oracle
    oracle.build()


_ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
