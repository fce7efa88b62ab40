import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def tiny_inputs():
    from block_sparse_video_reblock_amd import synth
    wl = synth.WORKLOADS["tiny_f32"]
    q, k, v = synth.make_qkv(wl)
    return wl, q[0].astype("float64"), k[0].astype("float64"), v[0].astype("float64")
