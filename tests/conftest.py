import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")
    config.addinivalue_line("markers", "slow: large shapes; minutes of CPU time")


_CONFIG_ORDER = ["tiny", "tiny_bf16", "ragged_f32", "ragged_bf16", "hd128_bf16", "chain_small",
                 "wide_bf16", "deep_bf16", "batch_bf16", "short_f32", "7b", "13b", "70b", "chain"]


def pytest_collection_modifyitems(session, config, items):
    """Run the parity tests config by config (their inputs are cached per
    config); other tests keep their places."""
    idx = [i for i, it in enumerate(items) if it.nodeid.startswith("tests/test_gpu_parity.py")]
    sub = [items[i] for i in idx]

    def key(it):
        cs = getattr(it, "callspec", None)
        name = cs.params.get("name") if cs is not None else None
        return _CONFIG_ORDER.index(name) if name in _CONFIG_ORDER else len(_CONFIG_ORDER)

    sub.sort(key=key)
    for i, it in zip(idx, sub):
        items[i] = it
