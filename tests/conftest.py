import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    # The oracle and the row generator are plain C built with gcc in seconds;
    # build them when missing so a fresh checkout can run the CPU suite.
    from oracle import build as obuild
    from workload import build as wbuild
    for mod in (obuild, wbuild):
        if not os.path.exists(mod.LIB):
            mod.build()
