import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_FULL = {}


@pytest.fixture(scope="session")
def full_layer():
    """The full-shape layer (hidden 4096, 256 experts, intermediate 2048) on the
    host and the device, generated once per session (about 3.4 GB each)."""
    if "layer" not in _FULL:
        import mxfp4_moe_expert_amd as mx
        import synth

        wl = synth.WORKLOADS["decode_t1"]
        print("[generating the full-shape layer]", flush=True)
        L = synth.make_layer(wl)
        _FULL["layer"] = L
        _FULL["dev"] = mx.DeviceLayer.from_host(L, "cuda")
    return _FULL["layer"], _FULL["dev"]
