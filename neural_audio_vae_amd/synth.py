"""Seeded synthetic inputs for the decoder: parameters, latents and the
per-channel de-normalization vectors.

This module only draws random numbers into named, shaped float32 arrays; it
holds none of the decoder's arithmetic and imports neither the GPU library
nor any reference implementation, so both can be fed from it.

Distributions (there are no released weights to load):

* conv weights ``v ~ N(0, 1) / sqrt(fan_in * k)``, fan_in being the weight's
  input channels (axis 0 for a transposed conv), with ``g`` set to the
  row norm of ``v`` so the folded weight keeps that distribution
  (``g_mode="norm"``); ``g_mode="uniform"`` draws ``g ~ U[0.5, 1.5]`` instead,
  which makes the fold change the weights;
* biases ``N(0, 0.01)`` (standard deviation 0.01);
* SnakeBeta ``alpha, beta ~ U[0.5, 1.5]`` per channel;
* latents ``N(0, 1)``; de-normalization ``std_c ~ U[0.5, 2]``,
  ``mean_c ~ N(0, 0.1)``.

Every stream is a numpy PCG64 generator keyed by ``(seed, stream, ...)``:
stream 0 parameters, 1 latents, 2 mean/std, 3 free-standing stage inputs,
4 encoder parameters (plain Snake ``alpha ~ U[0.5, 1.5]``), 5 waveforms
(``N(0, 0.25)``, clipped to [-1, 1]), 6 attention-projection and mean_proj
parameters.
The parameters therefore do not depend on the batch or sequence length.
"""

from __future__ import annotations

import numpy as np

DEFAULTS = {
    "latent_channels": 32,
    "latent_dim": 2048,
    "decoder_dim": 1024,
    "decoder_rates": (5, 5, 2, 2, 2, 2, 2),
    "decoder_kernel_sizes": (9, 9, 4, 4, 4, 4, 4),
    "resblock_kernel_sizes": (3, 7, 11),
    "resblock_dilation_sizes": ((1, 3, 5), (1, 3, 5), (1, 3, 5)),
}


def _cfg(config):
    c = dict(DEFAULTS)
    if config:
        c.update({k: v for k, v in config.items() if k in DEFAULTS})
    return c


def param_specs(config=None):
    """(name, shape, kind) for every decoder parameter, in a fixed order.
    kind is one of: w (plain weight), v (weight-norm direction, whose fan-in
    axis is given by the shape), g, bias, alpha, beta."""
    c = _cfg(config)
    specs = []
    lc, ld, dd = c["latent_channels"], c["latent_dim"], c["decoder_dim"]
    specs.append(("dec_in_proj.weight", (ld, lc, 1), "w"))
    specs.append(("dec_in_proj.bias", (ld,), "bias"))
    specs.append(("decoder.conv_pre.weight_v", (dd, ld, 7), "v"))
    specs.append(("decoder.conv_pre.weight_g", (dd, 1, 1), "g"))
    specs.append(("decoder.conv_pre.bias", (dd,), "bias"))
    ch = dd
    nrb = len(c["resblock_kernel_sizes"])
    for s, (r, k) in enumerate(zip(c["decoder_rates"], c["decoder_kernel_sizes"])):
        co = ch // 2
        specs.append((f"decoder.ups.{s}.0.weight_v", (ch, co, k), "vT"))
        specs.append((f"decoder.ups.{s}.0.weight_g", (ch, 1, 1), "g"))
        specs.append((f"decoder.ups.{s}.0.bias", (co,), "bias"))
        ch = co
        for j, (kk, dils) in enumerate(zip(c["resblock_kernel_sizes"], c["resblock_dilation_sizes"])):
            p = f"decoder.resblocks.{s * nrb + j}"
            for n in range(len(dils)):
                for conv in ("convs1", "convs2"):
                    specs.append((f"{p}.{conv}.{n}.weight_v", (ch, ch, kk), "v"))
                    specs.append((f"{p}.{conv}.{n}.weight_g", (ch, 1, 1), "g"))
                    specs.append((f"{p}.{conv}.{n}.bias", (ch,), "bias"))
            for m in range(2 * len(dils)):
                specs.append((f"{p}.activations.{m}.act.alpha", (ch,), "alpha"))
                specs.append((f"{p}.activations.{m}.act.beta", (ch,), "beta"))
    specs.append(("decoder.activation_post.act.alpha", (ch,), "alpha"))
    specs.append(("decoder.activation_post.act.beta", (ch,), "beta"))
    specs.append(("decoder.conv_post.weight_v", (1, ch, 7), "v"))
    specs.append(("decoder.conv_post.weight_g", (1, 1, 1), "g"))
    specs.append(("decoder.conv_post.bias", (1,), "bias"))
    return specs


def make_params(config=None, seed=0, g_mode="norm"):
    """Decoder parameters as a dict name -> float32 array (see module doc)."""
    rng = np.random.default_rng([seed, 0])
    out = {}
    last_v = None
    for name, shape, kind in param_specs(config):
        if kind in ("w", "v", "vT"):
            fan_in = shape[0] if kind == "vT" else shape[1]
            arr = rng.standard_normal(shape) / np.sqrt(fan_in * shape[2])
            last_v = arr
        elif kind == "g":
            if g_mode == "norm":
                arr = np.sqrt(np.sum(last_v * last_v, axis=(1, 2))).reshape(shape)
            elif g_mode == "uniform":
                arr = rng.uniform(0.5, 1.5, size=shape)
            else:
                raise ValueError(g_mode)
        elif kind == "bias":
            arr = rng.normal(0.0, 0.01, size=shape)
        elif kind in ("alpha", "beta"):
            arr = rng.uniform(0.5, 1.5, size=shape)
        else:
            raise AssertionError(kind)
        out[name] = np.ascontiguousarray(arr, dtype=np.float32)
    return out


def make_latents(batch, frames, seed=0, channels=32):
    """Latents (batch, channels, frames) ~ N(0, 1), float32."""
    rng = np.random.default_rng([seed, 1, batch, frames])
    return rng.standard_normal((batch, channels, frames)).astype(np.float32)


def make_denorm(channels=32, seed=0):
    """(latents_mean, latents_std): mean ~ N(0, 0.1), std ~ U[0.5, 2]."""
    rng = np.random.default_rng([seed, 2])
    mean = rng.normal(0.0, 0.1, size=channels).astype(np.float32)
    std = rng.uniform(0.5, 2.0, size=channels).astype(np.float32)
    return mean, std


def make_signal(shape, seed=0, scale=1.0):
    """A free-standing input tensor ~ N(0, scale^2), float32 (stage and
    layer tests)."""
    rng = np.random.default_rng([seed, 3] + [int(s) for s in shape])
    return (scale * rng.standard_normal(shape)).astype(np.float32)


ENC_DEFAULTS = {"encoder_dim": 64, "encoder_rates": (2, 4, 4, 5, 5), "latent_dim": 2048}


def encoder_param_specs(config=None):
    """(name, shape, kind) for every parameter of the encoder's convolution
    stack (the names ``MLXMiniMaxH3AudioVAE.encode`` reads)."""
    c = dict(ENC_DEFAULTS)
    if config:
        c.update({k: v for k, v in config.items() if k in ENC_DEFAULTS})
    specs = []

    def conv(prefix, c_out, c_in, k):
        specs.append((f"{prefix}.weight_v", (c_out, c_in, k), "v"))
        specs.append((f"{prefix}.weight_g", (c_out, 1, 1), "g"))
        specs.append((f"{prefix}.bias", (c_out,), "bias"))

    dim = c["encoder_dim"]
    conv("encoder.block.0", dim, 1, 7)
    for index, stride in enumerate(c["encoder_rates"], start=1):
        p = f"encoder.block.{index}"
        for unit in range(3):
            u = f"{p}.block.{unit}"
            specs.append((f"{u}.block.0.alpha", (dim,), "alpha"))
            conv(f"{u}.block.1", dim, dim, 7)
            specs.append((f"{u}.block.2.alpha", (dim,), "alpha"))
            conv(f"{u}.block.3", dim, dim, 1)
        specs.append((f"{p}.block.3.alpha", (dim,), "alpha"))
        conv(f"{p}.block.4", 2 * dim, dim, 2 * stride)
        dim *= 2
    n = len(c["encoder_rates"])
    specs.append((f"encoder.block.{n + 1}.alpha", (dim,), "alpha"))
    conv(f"encoder.block.{n + 2}", c["latent_dim"], dim, 3)
    return specs


def make_encoder_params(config=None, seed=0):
    """Encoder convolution-stack parameters, name -> float32 array (weights
    v ~ N(0, 1) / sqrt(fan_in k) with g = ||v|| per output channel, biases
    N(0, 0.01), alpha ~ U[0.5, 1.5])."""
    rng = np.random.default_rng([seed, 4])
    out = {}
    last_v = None
    for name, shape, kind in encoder_param_specs(config):
        if kind == "v":
            arr = rng.standard_normal(shape) / np.sqrt(shape[1] * shape[2])
            last_v = arr
        elif kind == "g":
            arr = np.sqrt(np.sum(last_v * last_v, axis=(1, 2))).reshape(shape)
        elif kind == "bias":
            arr = rng.normal(0.0, 0.01, size=shape)
        else:
            arr = rng.uniform(0.5, 1.5, size=shape)
        out[name] = np.ascontiguousarray(arr, dtype=np.float32)
    return out


def make_waveform(batch, samples, seed=0):
    """Waveforms (batch, 1, samples) ~ N(0, 0.25) clipped to [-1, 1], float32."""
    rng = np.random.default_rng([seed, 5, batch, samples])
    return np.clip(0.5 * rng.standard_normal((batch, 1, samples)), -1.0, 1.0).astype(np.float32)


PRE_DEFAULTS = {"latent_dim": 2048, "latent_channels": 32, "num_attention_heads": 8, "mlp_width": 128}
# q/k and v weights are N(0, 1) / sqrt(D) times these: the encoder's hidden
# state has an rms of ~120 under the synthetic encoder weights, so the
# attention scores then spread over a few units (neither uniform nor
# one-hot) and the GeGLU sees values of order one.
QK_SCALE, V_SCALE = 0.01, 0.1


def pre_block_param_specs(config=None):
    """(name, shape, kind) of the attention projection and mean_proj."""
    c = dict(PRE_DEFAULTS)
    if config:
        c.update({k: v for k, v in config.items() if k in PRE_DEFAULTS})
    d, lc, f = c["latent_dim"], c["latent_channels"], c["mlp_width"]
    return [
        ("pre_block.attn.qkv.weight", (3 * d, d), "qkv"),
        ("pre_block.attn.q_bias", (d,), "bias"),
        ("pre_block.attn.v_bias", (d,), "bias"),
        ("pre_block.attn.proj.weight", (lc, lc), "w"),
        ("pre_block.attn.proj.bias", (lc,), "bias"),
        ("pre_block.mlp.fc1.weight", (2 * f, lc), "w"),
        ("pre_block.mlp.fc1.bias", (2 * f,), "bias"),
        ("pre_block.mlp.fc2.weight", (lc, f), "w"),
        ("pre_block.mlp.fc2.bias", (lc,), "bias"),
        ("mean_proj.weight", (lc, lc, 1), "w"),
        ("mean_proj.bias", (lc,), "bias"),
    ]


def make_pre_block_params(config=None, seed=0):
    """Attention-projection and mean_proj parameters, name -> float32 array:
    linear weights N(0, 1) / sqrt(fan_in) (q, k times QK_SCALE, v times
    V_SCALE), biases N(0, 0.01)."""
    rng = np.random.default_rng([seed, 6])
    out = {}
    for name, shape, kind in pre_block_param_specs(config):
        if kind == "qkv":
            arr = rng.standard_normal(shape) / np.sqrt(shape[1])
            d = shape[0] // 3
            arr[:2 * d] *= QK_SCALE
            arr[2 * d:] *= V_SCALE
        elif kind == "w":
            arr = rng.standard_normal(shape) / np.sqrt(shape[1])
        else:
            arr = rng.normal(0.0, 0.01, size=shape)
        out[name] = np.ascontiguousarray(arr, dtype=np.float32)
    return out
