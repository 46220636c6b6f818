"""The released-checkpoint adapter on synthetic component directories
(no released weights exist here): key filtering, required tensors, the
fp32-only rule, config.json reading; on the GPU, a decoder and encoder
loaded from a checkpoint match ones built from the same arrays."""

import json
import os

import numpy as np
import pytest

from neural_audio_vae_amd import checkpoint, synth
from tests.conftest import SMALL_CONFIG

ENC_SMALL = {"encoder_dim": 4, "latent_dim": 16}
# the attention projection of that encoder: latent_channels must match the
# decoder's (4), two heads of 8 features
PRE_SMALL = {"latent_dim": 16, "latent_channels": 4, "num_attention_heads": 2, "mlp_width": 6}


def write_component(tmp_path, params, config=None, extra=None):
    from safetensors.numpy import save_file

    tensors = {k: np.ascontiguousarray(v) for k, v in params.items()}
    tensors.update(extra or {})
    save_file(tensors, os.fspath(tmp_path / checkpoint.WEIGHTS_FILE))
    if config is not None:
        (tmp_path / checkpoint.CONFIG_FILE).write_text(json.dumps(config))
    return tmp_path


@pytest.fixture(scope="module")
def dec_params():
    return synth.make_params(SMALL_CONFIG, seed=3)


def test_read_weights_keeps_the_model_prefixes(tmp_path, dec_params):
    extra = {"encoder.block.0.weight_v": np.ones((4, 1, 7), np.float32), "quant.x": np.zeros(3, np.float32),
             "mean_proj.weight": np.ones((2, 2, 1), np.float32)}
    d = write_component(tmp_path, dec_params, extra=extra)
    got = checkpoint.read_weights(d / checkpoint.WEIGHTS_FILE)
    assert set(got) == set(dec_params) | {"mean_proj.weight"}
    for k, v in dec_params.items():
        np.testing.assert_array_equal(got[k], v)


def test_read_weights_required_tensors(tmp_path, dec_params):
    p = dict(dec_params)
    del p["decoder.conv_post.weight_v"]
    d = write_component(tmp_path, p)
    with pytest.raises(KeyError, match="decoder.conv_post.weight_v"):
        checkpoint.read_weights(d / checkpoint.WEIGHTS_FILE)


def test_read_weights_encoder_requires_its_tensors(tmp_path, dec_params):
    enc = synth.make_encoder_params(ENC_SMALL, seed=1)
    d = write_component(tmp_path, dict(dec_params, **enc))
    with pytest.raises(KeyError, match="pre_block.attn.qkv.weight"):
        checkpoint.read_weights(d / checkpoint.WEIGHTS_FILE, include_encoder=True)
    extra = {"mean_proj.weight": np.ones((2, 2, 1), np.float32), "logs_proj.weight": np.ones((2, 2, 1), np.float32),
             "pre_block.attn.qkv.weight": np.ones((6, 2), np.float32)}
    d = write_component(tmp_path, dict(dec_params, **enc), extra=extra)
    got = checkpoint.read_weights(d / checkpoint.WEIGHTS_FILE, include_encoder=True)
    assert set(enc) <= set(got) and "pre_block.attn.qkv.weight" in got


def test_read_weights_rejects_non_fp32_storage(tmp_path, dec_params):
    p = dict(dec_params)
    p["decoder.conv_pre.bias"] = p["decoder.conv_pre.bias"].astype(np.float16)
    d = write_component(tmp_path, p)
    with pytest.raises(ValueError, match="float32"):
        checkpoint.read_weights(d / checkpoint.WEIGHTS_FILE)


def test_load_from_dir_checks_before_loading(tmp_path):
    with pytest.raises(ValueError, match="fp32"):
        checkpoint.load_from_dir(tmp_path, storage_dtype="bf16")
    with pytest.raises(FileNotFoundError):
        checkpoint.load_from_dir(tmp_path)


def test_read_config_keeps_constructor_keys(tmp_path):
    assert checkpoint.read_config(tmp_path) == {}
    cfg = dict(SMALL_CONFIG, decoder_rates=[5, 5, 2, 2, 2, 2, 2], latents_mean=None, _class_name="X", foo=3)
    (tmp_path / checkpoint.CONFIG_FILE).write_text(json.dumps(cfg))
    got = checkpoint.read_config(tmp_path)
    assert got == dict(SMALL_CONFIG, decoder_rates=[5, 5, 2, 2, 2, 2, 2])


@pytest.mark.gpu
def test_checkpoint_decoder_and_encoder_match_direct(tmp_path, dec_params):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from neural_audio_vae_amd import Decoder, Encoder
    enc_params = synth.make_encoder_params(dict(ENC_SMALL), seed=2)
    mean, std = synth.make_denorm(SMALL_CONFIG["latent_channels"])
    config = dict(SMALL_CONFIG, latents_mean=[float(v) for v in mean], latents_std=[float(v) for v in std],
                  **ENC_SMALL)
    extra = dict(synth.make_pre_block_params(PRE_SMALL, seed=2), **{"logs_proj.weight": np.ones((4, 4, 1), np.float32)})
    config["num_attention_heads"] = 2
    d = write_component(tmp_path, dict(dec_params, **enc_params), config=config, extra=extra)
    print("[case] checkpoint load + decode / encode vs direct", flush=True)
    dec, enc = checkpoint.load_from_dir(d, include_encoder=True)
    ref_dec = Decoder(dec_params, SMALL_CONFIG, latents_mean=mean, latents_std=std)
    ref_enc = Encoder(dict(enc_params, **extra), dict(ENC_SMALL, latent_channels=4, num_attention_heads=2))
    z = torch.from_numpy(synth.make_latents(2, 3, seed=1, channels=4)).cuda()
    np.testing.assert_array_equal(dec.decode(z, flags=0x1 | 0x4).cpu().numpy(),
                                  ref_dec.decode(z, flags=0x1 | 0x4).cpu().numpy())
    w = torch.from_numpy(synth.make_waveform(1, 2400, seed=1)).cuda()
    np.testing.assert_array_equal(enc.encode_hidden(w).cpu().numpy(), ref_enc.encode_hidden(w).cpu().numpy())
    np.testing.assert_array_equal(enc.encode_mean(w).cpu().numpy(), ref_enc.encode_mean(w).cpu().numpy())
    torch.cuda.synchronize()
    for o in (dec, enc, ref_dec, ref_enc):
        o.close()


@pytest.mark.gpu
def test_checkpoint_decoder_and_encoder_match_the_oracle(tmp_path, dec_params):
    # A component directory as the loader reads it (weights, config.json with
    # the de-normalization vectors, released filter buffers for two
    # activations): the loaded decoder and encoder against the oracle run on
    # the arrays that were written, with the config and vectors as written.
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle as O
    p = dict(dec_params)
    rng = np.random.default_rng(7)
    for name in ("decoder.resblocks.4.activations.3", "decoder.activation_post"):
        f = rng.uniform(-0.2, 0.6, size=12).astype(np.float32)
        p[name + ".upsample.filter"] = f
        p[name + ".downsample.lowpass.filter"] = np.ascontiguousarray(f[::-1])
    enc_params = synth.make_encoder_params(dict(ENC_SMALL), seed=2)
    mean, std = synth.make_denorm(SMALL_CONFIG["latent_channels"])
    config = dict(SMALL_CONFIG, latents_mean=[float(v) for v in mean], latents_std=[float(v) for v in std],
                  **ENC_SMALL)
    pre = synth.make_pre_block_params(PRE_SMALL, seed=3)
    extra = dict(pre, **{"logs_proj.weight": np.ones((4, 4, 1), np.float32)})
    config["num_attention_heads"] = 2
    d = write_component(tmp_path, dict(p, **enc_params), config=config, extra=extra)
    print("[case] checkpoint-loaded decoder / encoder vs the oracle", flush=True)
    dec, enc = checkpoint.load_from_dir(d, include_encoder=True)
    z = synth.make_latents(2, 9, seed=4, channels=SMALL_CONFIG["latent_channels"])
    got = dec.decode(torch.from_numpy(z).cuda(), flags=0x1 | 0x4).cpu().numpy().astype(np.float64)
    ref = O.decode(p, z, SMALL_CONFIG, denormalize=True, latents_mean=mean, latents_std=std,
                   clamp=False).astype(np.float64)
    rl = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    tol = 1e-3 * max(1.0, float(np.max(np.abs(ref))) / 10.0)
    print(f"[parity] checkpoint decode: rel_l2={rl:.3e} max_abs={np.max(np.abs(got - ref)):.3e}", flush=True)
    assert rl <= 1e-4 and np.max(np.abs(got - ref)) <= tol
    w = synth.make_waveform(2, 3 * 800 + 211, seed=3)
    h = enc.encode_hidden(torch.from_numpy(w).cuda()).cpu().numpy().astype(np.float64)
    href = O.encode_hidden(enc_params, w, ENC_SMALL).astype(np.float64)
    rl = float(np.linalg.norm(h - href) / np.linalg.norm(href))
    tol = 1e-3 * max(1.0, float(np.max(np.abs(href))) / 10.0)
    print(f"[parity] checkpoint encode: rel_l2={rl:.3e} max_abs={np.max(np.abs(h - href)):.3e}", flush=True)
    assert rl <= 1e-4 and np.max(np.abs(h - href)) <= tol
    # the posterior mean: stack, attention projection, mean_proj
    ocfg = dict(ENC_SMALL, latent_channels=4, num_attention_heads=2)
    mu = enc.encode_mean(torch.from_numpy(w).cuda()).cpu().numpy().astype(np.float64)
    muref = O.encode(dict(enc_params, **pre), w, ocfg).astype(np.float64)
    rl = float(np.linalg.norm(mu - muref) / np.linalg.norm(muref))
    print(f"[parity] checkpoint encode mean: rel_l2={rl:.3e} max_abs={np.max(np.abs(mu - muref)):.3e}", flush=True)
    assert rl <= 1e-4 and np.max(np.abs(mu - muref)) <= 1e-3
    torch.cuda.synchronize()
    dec.close()
    enc.close()
