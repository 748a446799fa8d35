import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # Tests marked gpu are skipped (not failed) when no GPU is present, so the
    # CPU suite can be run with or without -m "not gpu".
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
    # DA_PARITY_RECORD=path: write the largest errors of every GPU parity check
    path = os.environ.get("DA_PARITY_RECORD")
    if not path:
        return
    try:
        from gpu_util import RECORD
    except Exception:  # pragma: no cover  (no GPU test was collected)
        return
    import json
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "w") as f:
        json.dump(dict(exitstatus=int(exitstatus), checks=RECORD), f, indent=1, sort_keys=True)
