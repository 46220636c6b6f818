import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    config.addinivalue_line("markers", "full_oracle(*jobs): GPU test that compares a full-size workload with "
                                       "oracle results computed in background workers (tests/full_oracle.py)")


_FULL_ORACLE = None


def pytest_collection_finish(session):
    """Start the oracle workers for the selected full-size tests (only when
    such tests are selected and a GPU is there to run them)."""
    global _FULL_ORACLE
    names = []
    for item in session.items:
        m = item.get_closest_marker("full_oracle")
        if m:
            names += [n for n in m.args if n not in names]
    if not names:
        return
    try:
        import torch
        if torch.cuda.device_count() < 1:  # (counting devices does not initialise the GPU)
            return
    except Exception:
        return
    from tests.full_oracle import Pool
    _FULL_ORACLE = Pool(names)


def pytest_sessionfinish(session, exitstatus):
    global _FULL_ORACLE
    if _FULL_ORACLE is not None:
        _FULL_ORACLE.close()
        _FULL_ORACLE = None


@pytest.fixture(scope="session")
def full_oracle():
    if _FULL_ORACLE is None:
        pytest.skip("full-size oracle workers not started (no GPU)")
    return _FULL_ORACLE


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


def encoder_margin_frames(rates):
    """Frames of context on either side that make an encoder window's
    interior equal to the full encode: the stack's one-sided reach in samples
    (k7 first conv: 3; per block at sample spacing P: units of dilation 1, 3,
    9 reach 3 (1 + 3 + 9) = 39 positions, the strided conv p = ceil(s / 2)
    back and 2 s - 1 - p forward; final k3: one frame), plus one frame."""
    hop, P, left, right = 1, 1, 3, 3
    for s in rates:
        p = (s + 1) // 2
        left += (39 + p) * P
        right += (39 + 2 * s - 1 - p) * P
        P *= s
    hop = P
    left += hop
    right += hop
    return -(-max(left, right) // hop) + 1
