import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # the CPU-side libraries are built by __graft_entry__.build(); build them here
    # only when nothing is built yet (gcc, a few seconds)
    import oracle
    import synth
    if not os.path.exists(oracle.SO):
        oracle.build()
    if not os.path.exists(synth.HOST_SO):
        import subprocess
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", synth.HOST_SO, os.path.join(ROOT, "synth", "synth_host.c")])
