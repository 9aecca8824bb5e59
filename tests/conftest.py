"""pytest configuration: the ``gpu`` marker and shared helpers."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    pkg = os.path.join(ROOT, "quantized_kv_flashattention_amd")
    if not all(os.path.exists(os.path.join(pkg, n)) for n in ("libqkvfa.so", "libqkvfa_bench.so")):
        # nothing built yet: build once (hipcc cross-compiles without a GPU)
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "qkvfa_build", os.path.join(ROOT, "quantized_kv_flashattention_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
