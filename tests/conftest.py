import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # The whole-tensor parity checks run the fp64 oracle in a pool of spawned worker
    # processes. Start it before any test initialises the GPU, so that no worker is
    # created from a process that holds a GPU context (counting devices does not
    # initialise one).
    try:
        import torch
        has_gpu = torch.cuda.device_count() > 0
    except Exception:
        has_gpu = False
    if has_gpu:
        from oracle.fullcheck import start_pool
        start_pool()


def pytest_sessionfinish(session, exitstatus):
    from oracle import fullcheck
    if fullcheck._pool is not None:
        fullcheck._pool.terminate()
        fullcheck._pool.join()
