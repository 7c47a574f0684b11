import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


_spawner = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C ABI")
    # Started before anything initialises the GPU: a process that has must not
    # exec another program, so GPU programs that tests run as separate processes
    # are launched from this helper.
    global _spawner
    _spawner = subprocess.Popen([sys.executable, os.path.join(ROOT, "tests", "spawner.py")],
                                stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)


def pytest_unconfigure(config):
    if _spawner is not None and _spawner.poll() is None:
        _spawner.stdin.close()
        _spawner.wait(timeout=30)


@pytest.fixture(scope="session")
def run_program():
    """run_program(cmd, timeout) -> (rc, stdout, stderr), run from the GPU-free spawner process."""
    def run(cmd, timeout=120):
        _spawner.stdin.write(json.dumps({"cmd": [str(c) for c in cmd], "timeout": timeout}) + "\n")
        _spawner.stdin.flush()
        res = json.loads(_spawner.stdout.readline())
        return res["rc"], res["stdout"], res["stderr"]
    return run


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle


def _gpu_available():
    # device_count() does not initialise the GPU (is_available() does)
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
