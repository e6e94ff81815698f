import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def _ensure_built():
    """Build the HIP library and the oracle when nothing is built yet."""
    lib = os.path.join(ROOT, "quantized_moe_gemv_amd", "libmoegemv.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__._build_module().build()
    import oracle
    import qmoe_synth
    qmoe_synth._load()
    oracle.load()


_ensure_built()
