import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


def pytest_collection_modifyitems(session, config, items):
    # The full-size parity tests evaluate the oracle over every chain in worker
    # processes; they are spawned here, before any test initialises the GPU.
    if any(item.get_closest_marker("gpu") for item in items) and \
            os.environ.get("FALCON_ORACLE_POOL", "1") != "0":
        import oracle_pool
        oracle_pool.start()


def pytest_sessionfinish(session, exitstatus):
    mod = sys.modules.get("oracle_pool")
    if mod is not None:
        mod.stop()
