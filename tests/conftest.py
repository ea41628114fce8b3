import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    """Start the oracle pool's fork server while this process has not touched
    the GPU yet (the full-size parity tests fork their workers from it); only
    when GPU tests are selected."""
    expr = session.config.getoption("markexpr", default="") or ""
    if "not gpu" in expr.replace("  ", " "):
        return
    import oracle_pool
    oracle_pool.start_server()
