"""The C-ABI library loads, exports every symbol include/mh3a.h declares,
and rejects bad arguments before touching the GPU (no compute calls here)."""

import os
import re
import subprocess

import numpy as np
import pytest

from neural_audio_vae_amd import _lib, synth
from tests.conftest import ROOT, SMALL_CONFIG

HEADER = os.path.join(ROOT, "include", "mh3a.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mh3a_\w+)\s*\(", text)))


def test_library_exists_and_loads():
    assert os.path.exists(_lib.LIB_PATH), "build the library first: python -m neural_audio_vae_amd.build"
    _lib.load()


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(line.split()[-1] for line in out.stdout.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(_lib.EXPORTED)
    lib = _lib.load()
    for n in names:
        assert getattr(lib, n) is not None


def test_config_default_matches_constructor_defaults():
    # diffusers "AutoencoderKLMiniMaxH3Audio" constructor defaults
    c = _lib.mh3a_config_default()
    assert (c.latent_channels, c.latent_dim, c.decoder_dim, c.hop_length) == (32, 2048, 1024, 800)
    assert c.num_ups == 7
    assert list(c.rates[:7]) == [5, 5, 2, 2, 2, 2, 2]
    assert list(c.kernels[:7]) == [9, 9, 4, 4, 4, 4, 4]
    assert c.num_resblocks == 3 and list(c.rb_kernels[:3]) == [3, 7, 11]
    assert c.num_dilations == 3 and all(list(c.rb_dilations[j][:3]) == [1, 3, 5] for j in range(3))
    assert c.filter_taps == 12 and c.filter_cutoff == 0.25 and c.filter_half_width == 0.3


def test_make_config_overrides():
    c = _lib.make_config(SMALL_CONFIG)
    assert (c.latent_channels, c.latent_dim, c.decoder_dim) == (4, 16, 128)
    c = _lib.make_config({"decoder_rates": (4, 2), "decoder_kernel_sizes": (8, 4)})
    assert c.num_ups == 2 and c.hop_length == 8


@pytest.fixture(scope="module")
def small():
    return synth.make_params(SMALL_CONFIG, seed=3)


def create(cfg, params, mean=None, std=None, device=0):
    return _lib.mh3a_decoder_create(cfg, params, mean, std, device)


def expect_error(code, fn, *args, match=None):
    with pytest.raises(_lib.MH3AError) as e:
        fn(*args)
    assert e.value.code == code, str(e.value)
    if match:
        assert re.search(match, str(e.value)), str(e.value)


def test_create_rejects_null_config():
    lib = _lib.load()
    from ctypes import byref, c_void_p
    h = c_void_p()
    assert lib.mh3a_decoder_create(None, None, 0, None, None, 0, byref(h)) == _lib.MH3A_E_INVALID_ARG
    assert h.value is None
    assert lib.mh3a_decoder_create(None, None, 0, None, None, 0, None) == _lib.MH3A_E_INVALID_ARG


def test_create_missing_required_tensors(small):
    cfg = _lib.make_config(SMALL_CONFIG)
    for name in ("dec_in_proj.weight", "decoder.conv_pre.weight_v", "decoder.conv_post.weight_v"):
        p = dict(small)
        del p[name]
        expect_error(_lib.MH3A_E_MISSING_TENSOR, create, cfg, p, match=re.escape(name))
    p = dict(small)
    del p["decoder.resblocks.4.activations.3.act.beta"]
    expect_error(_lib.MH3A_E_MISSING_TENSOR, create, cfg, p, match="activations.3.act.beta")


def test_create_rejects_wrong_shapes(small):
    cfg = _lib.make_config(SMALL_CONFIG)
    p = dict(small)
    p["decoder.ups.2.0.weight_v"] = np.zeros((16, 16, 4), dtype=np.float32)
    expect_error(_lib.MH3A_E_SHAPE, create, cfg, p, match="ups.2.0.weight_v")
    p = dict(small)
    p["decoder.resblocks.0.convs1.0.bias"] = np.zeros(3, dtype=np.float32)
    expect_error(_lib.MH3A_E_SHAPE, create, cfg, p)
    p = dict(small)
    p["decoder.activation_post.upsample.filter"] = np.zeros(11, dtype=np.float32)
    expect_error(_lib.MH3A_E_SHAPE, create, cfg, p, match="upsample.filter")


def test_create_rejects_bad_configs(small):
    cfg = _lib.make_config(dict(SMALL_CONFIG, resblock_kernel_sizes=(), resblock_dilation_sizes=()))
    expect_error(_lib.MH3A_E_CONFIG, create, cfg, small, match="no residual blocks")
    cfg = _lib.make_config(SMALL_CONFIG)
    cfg.hop_length = 640
    expect_error(_lib.MH3A_E_CONFIG, create, cfg, small, match="product of decoder rates")
    cfg = _lib.make_config(SMALL_CONFIG)
    cfg.filter_taps = 10
    expect_error(_lib.MH3A_E_CONFIG, create, cfg, small)
    cfg = _lib.make_config(dict(SMALL_CONFIG, resblock_kernel_sizes=(3, 4, 11)))
    expect_error(_lib.MH3A_E_CONFIG, create, cfg, small, match="odd")
    cfg = _lib.make_config(SMALL_CONFIG)
    cfg.decoder_dim = 100
    expect_error(_lib.MH3A_E_CONFIG, create, cfg, small)


def test_create_rejects_negative_device(small):
    expect_error(_lib.MH3A_E_INVALID_ARG, create, _lib.make_config(SMALL_CONFIG), small, None, None, -1)


def test_decode_entry_points_reject_null_handles():
    lib = _lib.load()
    from ctypes import byref, c_int64, c_size_t
    n = c_size_t(123)
    assert lib.mh3a_decode_workspace_size(None, 1, 4, 0, byref(n)) == _lib.MH3A_E_INVALID_ARG and n.value == 0
    assert lib.mh3a_decode(None, None, 1, 4, None, None, 0, 0, None) == _lib.MH3A_E_INVALID_ARG
    assert lib.mh3a_decode_partial(None, None, 1, 4, 0, None, None, 0, 0, None) == _lib.MH3A_E_INVALID_ARG
    c, ln = c_int64(), c_int64()
    assert lib.mh3a_decode_layer_shape(None, 4, 0, byref(c), byref(ln)) == _lib.MH3A_E_INVALID_ARG
    assert lib.mh3a_amp_stage_workspace_size(None, 0, 1, 4, byref(n)) == _lib.MH3A_E_INVALID_ARG
    assert lib.mh3a_amp_stage(None, 0, None, 1, 4, None, None, 0, 0, None) == _lib.MH3A_E_INVALID_ARG
    assert _lib.mh3a_last_error() != ""
    lib.mh3a_destroy(None)  # no-op


def test_valid_create_reaches_the_device_step(small):
    # Every host step (lookup, weight-norm fold, filter design, packing)
    # succeeds; without a GPU the first HIP call reports MH3A_E_HIP.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    expect_error(_lib.MH3A_E_HIP, create, _lib.make_config(SMALL_CONFIG), small)


# ---- encoder convolution stack ----

ENC_SMALL = {"encoder_dim": 4, "latent_dim": 16}


def test_encoder_config_default():
    # the FastVideo encoder's defaults: encoder_dim 64, rates (2, 4, 4, 5, 5), latent_dim 2048
    c = _lib.mh3a_encoder_config_default()
    assert (c.encoder_dim, c.num_blocks, c.latent_dim) == (64, 5, 2048)
    assert list(c.rates[:5]) == [2, 4, 4, 5, 5]
    c = _lib.make_encoder_config({"encoder_dim": 8, "encoder_rates": (2, 2)})
    assert (c.encoder_dim, c.num_blocks, list(c.rates[:2])) == (8, 2, [2, 2])


@pytest.fixture(scope="module")
def enc_small():
    return synth.make_encoder_params(ENC_SMALL, seed=1)


def test_encoder_create_errors(enc_small):
    cfg = _lib.make_encoder_config(ENC_SMALL)
    for name in ("encoder.block.0.weight_v", "encoder.block.3.block.1.block.2.alpha", "encoder.block.7.bias"):
        p = dict(enc_small)
        del p[name]
        expect_error(_lib.MH3A_E_MISSING_TENSOR, _lib.mh3a_encoder_create, cfg, p, match=re.escape(name))
    p = dict(enc_small)
    p["encoder.block.2.block.4.weight_v"] = np.zeros((16, 8, 7), dtype=np.float32)
    expect_error(_lib.MH3A_E_SHAPE, _lib.mh3a_encoder_create, cfg, p, match="block.2.block.4.weight_v")
    p = dict(enc_small)
    p["encoder.block.1.block.0.block.0.alpha"] = np.ones(5, dtype=np.float32)
    expect_error(_lib.MH3A_E_SHAPE, _lib.mh3a_encoder_create, cfg, p)
    bad = _lib.make_encoder_config(ENC_SMALL)
    bad.num_blocks = 0
    expect_error(_lib.MH3A_E_CONFIG, _lib.mh3a_encoder_create, bad, enc_small)
    bad = _lib.make_encoder_config(ENC_SMALL)
    bad.rates[1] = 0
    expect_error(_lib.MH3A_E_CONFIG, _lib.mh3a_encoder_create, bad, enc_small)


def test_encoder_null_handle_errors():
    lib = _lib.load()
    from ctypes import byref, c_int64, c_size_t
    n = c_size_t()
    assert lib.mh3a_encode_workspace_size(None, 1, 800, 0, byref(n)) == _lib.MH3A_E_INVALID_ARG
    f = c_int64()
    assert lib.mh3a_encode_frames(None, 800, byref(f)) == _lib.MH3A_E_INVALID_ARG
    assert lib.mh3a_encode_hidden(None, None, 1, 800, None, None, 0, 0, None) == _lib.MH3A_E_INVALID_ARG
    lib.mh3a_encoder_destroy(None)


def test_matrix_form_defaults_and_checks(small):
    # the decoder and the encoder default to fp16 pieces; an unknown form is
    # a config error, raised before any HIP call
    assert _lib.mh3a_config_default().matrix_form == _lib.MH3A_MATRIX_SPLIT_F16
    assert _lib.mh3a_encoder_config_default().matrix_form == _lib.MH3A_MATRIX_SPLIT_F16
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decoder_create(_lib.make_config(dict(SMALL_CONFIG, matrix_form=7)), small)
    assert e.value.code == _lib.MH3A_E_CONFIG
    enc = synth.make_encoder_params({"encoder_dim": 4, "latent_dim": 16}, seed=1)
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_encoder_create(_lib.make_encoder_config({"encoder_dim": 4, "latent_dim": 16,
                                                          "matrix_form": 7}), enc)
    assert e.value.code == _lib.MH3A_E_CONFIG
