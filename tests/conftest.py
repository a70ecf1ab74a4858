import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) where there is no GPU, so that a
    # plain `pytest` on a CPU-only machine runs the CPU suite; on a GPU machine
    # `-m gpu` runs them and they fail loudly if the library is missing.
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


@pytest.fixture(scope="session")
def k3_layer():
    """The K3-shaped layer (seed 0) in HBM, shared by the GPU tests of a session."""
    import torch
    from layer_inputs import device_weights
    from synth import CONFIGS
    print("[fixture] generating the K3-shaped layer (seed 0) on the device", flush=True)
    w = device_weights(CONFIGS["k3_b1"], 0)
    yield w
    del w
    torch.cuda.empty_cache()


@pytest.fixture(scope="session")
def k3_stack():
    """The 8-layer decode-step stack (seed 0): MoE layers and dense blocks in HBM."""
    import torch
    from layer_inputs import dense_device, device_weights
    from memory_bound_mxfp4_amd.stack import DecodeStack
    from synth import CONFIGS
    cfg = CONFIGS["k3_stack8"]
    print("[fixture] generating the 8-layer stack (seed 0) on the device", flush=True)
    layers = [device_weights(cfg, 0, layer=l) for l in range(cfg.layers)]
    dense = [dense_device(cfg, 0, l) for l in range(cfg.layers)]
    stack = DecodeStack(layers, dense, cfg.batch, cfg.rms_eps)
    yield stack
    del stack, layers, dense
    torch.cuda.empty_cache()
