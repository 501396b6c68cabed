import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # the C oracle is compiled (if stale) before any test touches the GPU: a
    # process that has initialised the GPU must not start other programs
    from oracle import gemm as og
    og.build()
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run through the C-ABI library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")

