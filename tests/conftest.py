import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle work")


def pytest_collection_finish(session):
    # The GPU tests compare full-size outputs with the CPU oracle on several host processes.
    # Their forkserver starts here, before any test initialises the GPU, so no process holding
    # GPU state is forked.
    if any(item.get_closest_marker("gpu") for item in session.items):
        from oracle import pool as oracle_pool

        oracle_pool.start()
