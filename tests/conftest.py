import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_LIB = os.path.join(ROOT, "paged_kv_cache_indirected_amd", "libpkv.so")
_ORACLE = os.path.join(ROOT, "oracle", "liboracle.so")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # Build what is missing; never rebuild what exists, so the tests run the
    # libraries already built in this tree.
    if not os.path.exists(_ORACLE):
        import oracle
        oracle.build()
    if not os.path.exists(_LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_pkv_build", os.path.join(ROOT, "paged_kv_cache_indirected_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def pytest_collection_modifyitems(config, items):
    gpu_ok = None
    for item in items:
        if "gpu" in item.keywords:
            if gpu_ok is None:
                import torch
                gpu_ok = torch.cuda.is_available()
            if not gpu_ok:
                item.add_marker(pytest.mark.skip(reason="no GPU visible"))
