"""Released-checkpoint adapter: a component directory (config.json and one
safetensors file) -> Decoder / Encoder.

What it follows (FastVideo API docs "minimax_h3_audio_vae"):
  mlx_h3_audio_vae_from_dir: storage must be fp32; the weights are the single
    file diffusion_pytorch_model.safetensors under the component directory.
  mlx_h3_audio_vae_from_file: only tensors under the dec_in_proj., decoder.,
    mean_proj. and logs_proj. prefixes are kept (plus encoder. and pre_block.
    with the encoder), and the required tensors are checked: the decoder's
    dec_in_proj.weight, decoder.conv_pre.weight_v, decoder.conv_post.weight_v;
    with the encoder also mean_proj.weight, logs_proj.weight,
    pre_block.attn.qkv.weight and encoder.block.0.weight_v.
  MiniMaxH3AudioVAEConfigView: the architecture constants, named as the
    diffusers AutoencoderKLMiniMaxH3Audio constructor names them (class
    signature on the diffusers page), defaults for absent keys.
The checkpoint keys are the names the decode and encode sources read, so they
reach the library unchanged; released resampler filters
(<act>.upsample.filter, <act>.downsample.lowpass.filter) are used when
present. Every tensor must be stored as float32: the library computes on the
stored values and never converts.

Host-side file reading only: the numbers go to the library as they are.
"""

from __future__ import annotations

import json
import os

WEIGHTS_FILE = "diffusion_pytorch_model.safetensors"
CONFIG_FILE = "config.json"

# constructor keyword names (diffusers "AutoencoderKLMiniMaxH3Audio")
CONFIG_KEYS = (
    "encoder_dim", "encoder_rates", "latent_dim", "latent_channels", "num_attention_heads", "decoder_dim",
    "decoder_rates", "decoder_kernel_sizes", "resblock_kernel_sizes", "resblock_dilation_sizes", "sampling_rate",
    "latents_mean", "latents_std",
)
DECODER_PREFIXES = ("dec_in_proj.", "decoder.", "mean_proj.", "logs_proj.")
ENCODER_PREFIXES = ("encoder.", "pre_block.")
DECODER_REQUIRED = ("dec_in_proj.weight", "decoder.conv_pre.weight_v", "decoder.conv_post.weight_v")
ENCODER_REQUIRED = ("mean_proj.weight", "logs_proj.weight", "pre_block.attn.qkv.weight", "encoder.block.0.weight_v")


def read_config(component_dir):
    """The architecture constants in component_dir/config.json (only the
    constructor's keys; {} when the file is absent)."""
    path = os.path.join(os.fspath(component_dir), CONFIG_FILE)
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        raw = json.load(f)
    if not isinstance(raw, dict):
        raise ValueError(f"{path}: expected a JSON object")
    return {k: raw[k] for k in CONFIG_KEYS if k in raw and raw[k] is not None}


def read_weights(weights_path, include_encoder=False):
    """name -> float32 numpy array for the tensors the model keeps. Raises
    KeyError naming the missing required tensors and ValueError for a
    tensor not stored as float32."""
    from safetensors import safe_open

    prefixes = DECODER_PREFIXES + (ENCODER_PREFIXES if include_encoder else ())
    out = {}
    with safe_open(os.fspath(weights_path), framework="numpy") as f:
        for key in f.keys():
            if not key.startswith(prefixes):
                continue
            arr = f.get_tensor(key)
            if str(arr.dtype) != "float32":
                raise ValueError(f"{key} is stored as {arr.dtype}; the audio VAE needs float32 storage")
            out[key] = arr
    required = DECODER_REQUIRED + (ENCODER_REQUIRED if include_encoder else ())
    missing = [k for k in required if k not in out]
    if missing:
        raise KeyError(f"audio VAE checkpoint is missing required tensors: {missing}")
    return out


def load_from_file(weights_path, include_encoder=False, config=None, component_dir=None, device=0):
    """(Decoder, Encoder or None) from one safetensors file; config from
    `config` or else component_dir's (default: the file's directory)
    config.json."""
    from .decoder import Decoder, Encoder

    if config is None:
        config = read_config(component_dir if component_dir is not None else os.path.dirname(os.fspath(weights_path)))
    config = dict(config)
    params = read_weights(weights_path, include_encoder)
    dec_cfg = {k: v for k, v in config.items() if k not in ("latents_mean", "latents_std")}
    dec = Decoder(params, dec_cfg, latents_mean=config.get("latents_mean"), latents_std=config.get("latents_std"),
                  device=device)
    enc = None
    if include_encoder:
        enc_cfg = {k: config[k] for k in ("encoder_dim", "encoder_rates", "latent_dim", "latent_channels",
                                          "num_attention_heads") if k in config}
        enc = Encoder(params, enc_cfg, device=device)
    return dec, enc


def load_from_dir(component_dir, include_encoder=False, storage_dtype="fp32", device=0):
    """(Decoder, Encoder or None) from a released component directory."""
    if storage_dtype != "fp32":
        raise ValueError(f"the audio VAE needs storage_dtype='fp32', got {storage_dtype!r}")
    path = os.path.join(os.fspath(component_dir), WEIGHTS_FILE)
    if not os.path.exists(path):
        raise FileNotFoundError(f"no audio VAE safetensors under {component_dir}")
    return load_from_file(path, include_encoder=include_encoder, component_dir=component_dir, device=device)
