import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # load what is built; build only when nothing is
    pkg = os.path.join(ROOT, "communication_tensor_gemm_amd")
    lib = os.path.join(pkg, "libdistgemm.so")
    if os.path.isdir(pkg) and not os.path.exists(lib):
        # by path: importing the package needs the library that is missing
        import importlib.util
        spec = importlib.util.spec_from_file_location("_distgemm_build", os.path.join(pkg, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


def pytest_collection_modifyitems(config, items):
    # GPU tests are opt-in through -m gpu; without a GPU they are skipped, not failed.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
