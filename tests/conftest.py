import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_LIBS = [
    os.path.join(ROOT, "oracle", "liboracle.so"),
    os.path.join(ROOT, "synth", "libsynth_host.so"),
    os.path.join(ROOT, "synth", "libsynth_dev.so"),
    os.path.join(ROOT, "zero_partitioned_mixed_plan_amd", "libzero_mi355x.so"),
]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    if not all(os.path.exists(p) for p in _LIBS):
        import __graft_entry__
        __graft_entry__.build()
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    if tests_dir not in sys.path:
        sys.path.insert(0, tests_dir)
    import harness
    harness.CAPTURE_MANAGER = config.pluginmanager.getplugin("capturemanager")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    # release the library's plans and pipelines before interpreter shutdown
    z = sys.modules.get("zero_partitioned_mixed_plan_amd")
    if z is not None:
        z.release_all()
