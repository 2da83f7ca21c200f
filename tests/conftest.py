import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # Build only what is missing: tests load what is built.
    import __graft_entry__ as ge
    if not os.path.exists(os.path.join(ROOT, "oracle", "libhy_oracle.so")):
        ge.build_oracle()
    if not (os.path.exists(os.path.join(ROOT, "hy_inputs", "libhy_gen.so"))
            and os.path.exists(os.path.join(ROOT, "hy_inputs", "libhy_gen_dev.so"))):
        ge.build_inputs()
    pkg = os.path.join(ROOT, "sparse_moe_transformer_route_amd")
    if os.path.exists(os.path.join(pkg, "_build.py")) and not os.path.exists(os.path.join(pkg, "libhy_moe.so")):
        from sparse_moe_transformer_route_amd import _build
        _build.build()


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
