import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def default_params():
    from neural_audio_vae_amd import synth
    return synth.make_params()


# A narrow decoder (same structure, small widths) for structural checks that
# need several full decodes.
SMALL_CONFIG = {
    "latent_channels": 4,
    "latent_dim": 16,
    "decoder_dim": 128,
}


@pytest.fixture(scope="session")
def small_params():
    from neural_audio_vae_amd import synth
    return synth.make_params(SMALL_CONFIG, seed=3)
