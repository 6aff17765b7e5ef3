import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # the sanitizer tier (tests/test_sanitizers.py) reruns CPU suites against instrumented builds
    san = os.environ.get("RVQ_SANITIZED_DIR")
    if san:
        import oracle
        import synth
        from rvq_quantized_moe_amd import _lib
        _lib.LIB_PATH = os.path.join(san, "librvq.so")
        oracle._SO = os.path.join(san, "liboracle_san.so")
        synth._SO = os.path.join(san, "libsynth_san.so")


def pytest_sessionfinish(session, exitstatus):
    san = os.environ.get("RVQ_SANITIZED_DIR")
    if san:
        mapped = sorted({line.split()[-1] for line in open("/proc/self/maps") if san in line})
        print(f"\nsanitized builds mapped: {' '.join(os.path.basename(m) for m in mapped)}", file=sys.stderr)


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
