"""Plain CPU oracle for the MiniMax-H3 audio-VAE BigVGAN decoder.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the
package's smoke check and the CPU-baseline leg of the benchmark may import
this module. The GPU library never calls it and shares no code with it.

What it computes is the decode path described on two pages:

* diffusers docs, "AutoencoderKLMiniMaxH3Audio": the constructor defaults
  (section "AutoencoderKLMiniMaxH3Audio", parameter list) and the decode
  contract (section "decode": de-normalized latents (B, 32, N) in, waveform
  (B, 1, 800 N) out, clamped to [-1, 1]).
* FastVideo API docs, "minimax_h3_audio_vae": the module overview (BigVGAN
  decoder, weight-normalized ConvTranspose1d upsampling, AMP residual blocks
  with SnakeBeta behind alias-free Kaiser-window up/down sampling, final
  SnakeBeta, conv and clamp), the source of ``MLXMiniMaxH3AudioVAE.decode``
  (the order of the ops and their paddings) and ``kaiser_sinc_filter1d``
  (the low-pass design).

Numerics. The pages fix fp32 storage (``mlx_h3_audio_vae_from_dir`` refuses
anything but fp32, and the module overview gives waveforms as float32), so
every tensor between ops is float32. Inside each op the arithmetic is float64 and the op's output is
rounded to float32 once. Nothing is blocked, fused or reordered beyond what
each definition states; numpy's float64 matmul serves as the inner sum of a
convolution tap.

Readings of what the pages leave open:

* R1 ``_conv1d`` / ``_conv_transpose1d`` bodies are not shown: the standard
  PyTorch definitions (cross-correlation, zero padding, no output padding).
* R2 ``_wn_weight(v, g)``: w = g * v / ||v||, the norm over every axis but
  axis 0 of the stored weight (C_out for conv, C_in for transposed conv).
* R3 AMP block internals are not shown: BigVGAN's AMPBlock1 -- for each
  dilation d: x <- x + conv_{k,1}(act(conv_{k,d}(act(x)))), "same" zero
  padding d(k-1)/2, six activations per block.
* R4 the anti-aliased activation: BigVGAN's Activation1d -- 2x upsample
  (replicate pad 5, zero-insert transposed conv with the 12-tap filter,
  gain 2, crop 15/15), SnakeBeta at the 2x rate, 12-tap low-pass with
  replicate pad 5 left / 6 right and stride 2. Filter: cutoff 0.25,
  half-width 0.3, 12 taps.
* R5 SnakeBeta: y = x + sin^2(alpha x) / beta, alpha and beta per channel,
  used as stored (no log scale, no epsilon).
* R6 de-normalization, optional: z * std_c + mean_c (the convention the
  diffusers "AutoencoderKLMiniMaxH3" page states for its latents).
* R7 ``decoder.conv_post.bias`` is read with ``w.get``: absent means zero.

The encoder's convolution stack (``encode_hidden``: everything of
``MLXMiniMaxH3AudioVAE.encode`` before the attention projection) follows
the source of ``encode`` on the FastVideo page, with these readings:

* E1 ``_snake(x, alpha)`` is not shown: the plain Snake
  y = x + sin^2(alpha x) / (alpha + 1e-9), alpha per channel (the module
  overview calls the encoder's residual units plain-Snake).
* E2 the strided convolution's kernel is 2 x stride (not shown; the page
  gives its stride and padding ceil(stride / 2)); the residual units'
  second convolution has kernel 1 (no padding given); the final
  convolution has kernel 3 (padding 1) and latent_dim output channels.
* E3 the crop ``x[..., pad:-pad]`` never fires: every unit keeps the
  length ("same" padding), so pad = 0.

The attention projection ``pre_block`` and the posterior mean
(``encode_item``) follow the Encoder bullet of the FastVideo module
overview, which describes the block in prose only (causal multi-head
attention over the latent stream with q/v biases and a forced zero k bias,
head averaging, average pooling into latent_channels streams, an output
projection and a GeGLU MLP), the source of ``encode`` (the block runs on the
hidden state laid out time-major, then ``mean_proj`` is a 1x1 conv with
bias) and the diffusers page (``is_causal=True`` through the attention
dispatcher; ``num_attention_heads`` 8; ``latent_channels`` is the width of
``mean_proj``; the pipeline consumes only the posterior mean, never
``logs_proj``). Readings:

* P1 tokens are the N hidden frames, each a D = latent_dim vector; one
  fused projection ``pre_block.attn.qkv.weight`` (3D, D) gives q, k, v (in
  that order, the page's required tensor name) plus a bias (b_q, 0, b_v):
  the q and v biases are ``pre_block.attn.q_bias`` / ``v_bias`` (or the q
  and v thirds of a fused ``qkv.bias``), the k bias is zero whatever is
  stored.
* P2 H = num_attention_heads heads of hd = D / H consecutive features;
  scores q_t . k_u / sqrt(hd) (the scaled-dot-product default), causal:
  token t attends to u <= t; softmax over u; o_h[t] = sum_u p v_u.
* P3 head averaging: o[t] = (1 / H) sum_h o_h[t], a vector of hd.
* P4 average pooling into C = latent_channels streams: stream c is the
  mean of the g = hd / C consecutive features [c g, (c + 1) g).
* P5 output projection ``pre_block.attn.proj`` (C -> C, bias).
* P6 GeGLU MLP: ``pre_block.mlp.fc1`` (C -> 2F, bias) whose first half is
  the value and second half the gate, value * GELU(gate) with the exact
  (erf) GELU, then ``pre_block.mlp.fc2`` (F -> C, bias); F from the
  weights' shapes.
* P7 the steps compose in the order listed, with no residual connection
  and no normalization (none is named).
* P8 mean = ``mean_proj`` (1x1 conv, C -> latent_channels, bias) of the
  block's output laid out channels-first again.
"""

from __future__ import annotations

import math

import numpy as np

F32 = np.float32
F64 = np.float64

# Constructor defaults: diffusers "AutoencoderKLMiniMaxH3Audio", parameter
# list; the same values as FastVideo's MiniMaxH3AudioVAEConfigView.
DEFAULT_CONFIG = {
    "latent_channels": 32,
    "latent_dim": 2048,
    "decoder_dim": 1024,
    "decoder_rates": (5, 5, 2, 2, 2, 2, 2),
    "decoder_kernel_sizes": (9, 9, 4, 4, 4, 4, 4),
    "resblock_kernel_sizes": (3, 7, 11),
    "resblock_dilation_sizes": ((1, 3, 5), (1, 3, 5), (1, 3, 5)),
    "sampling_rate": 32000,
    "hop_length": 800,
    "encoder_dim": 64,
    "encoder_rates": (2, 4, 4, 5, 5),
    "num_attention_heads": 8,
    # Reading R4: BigVGAN's resampler, ratio 2.
    "filter_taps": 12,
    "filter_cutoff": 0.25,
    "filter_half_width": 0.3,
}


def _f32(a):
    return np.asarray(a, dtype=F64).astype(F32)


# ---------------------------------------------------------------------------
# Kaiser-windowed sinc low-pass of the anti-aliased activation: FastVideo
# "minimax_h3_audio_vae", the filter design of the Activation1d up/down
# samplers (kaiser_sinc_filter1d), from Kaiser's published design rules.
# ---------------------------------------------------------------------------

def bessel_i0(x):
    """Modified Bessel function of the first kind, order 0, by its power
    series sum_m ((x/2)^m / m!)^2, summed until the terms stop mattering."""
    x = np.asarray(x, dtype=F64)
    q = (x / 2.0) ** 2
    term = np.ones_like(x)
    total = np.ones_like(x)
    for m in range(1, 200):
        term = term * q / (m * m)
        total = total + term
        if np.all(term <= 1e-17 * total):
            break
    return total


def kaiser_attenuation(numtaps, width):
    """Kaiser's empirical length rule for a Kaiser-window FIR low-pass of
    numtaps taps and transition width `width` (a fraction of the Nyquist
    band), solved for the stop-band attenuation in dB:
    A = 7.95 + 2.285 (numtaps - 1) pi width (J. F. Kaiser, "Nonrecursive
    digital filter design using the I0-sinh window function", 1974)."""
    return 7.95 + 2.285 * (numtaps - 1) * math.pi * width


def kaiser_beta_for(attenuation):
    """Kaiser's shape parameter for a stop-band attenuation of A dB (same
    source; the Kaiser-window design rule in Oppenheim and Schafer,
    Discrete-Time Signal Processing): 0 below 21 dB, then
    0.5842 (A - 21)^0.4 + 0.07886 (A - 21) up to 50 dB, then
    0.1102 (A - 8.7)."""
    a = attenuation
    if a < 21.0:
        return 0.0
    if a <= 50.0:
        return 0.5842 * (a - 21.0) ** 0.4 + 0.07886 * (a - 21.0)
    return 0.1102 * (a - 8.7)


def kaiser_beta(cutoff, half_width, kernel_size):
    """The beta of the pages' anti-aliasing low-pass: Kaiser's rules above
    with the released filter's two readings of them, the length taken as
    kernel_size // 2 (not kernel_size) and the width as 4 * half_width.
    The cutoff does not enter."""
    return kaiser_beta_for(kaiser_attenuation(kernel_size // 2, 4.0 * half_width))


def kaiser_window(n, beta):
    """Symmetric Kaiser window of n points: I0(beta sqrt(1 - (2k/(n-1) - 1)^2)) / I0(beta)."""
    if n == 1:
        return np.ones(1, dtype=F64)
    k = np.arange(n, dtype=F64)
    r = 2.0 * k / (n - 1) - 1.0
    return bessel_i0(beta * np.sqrt(np.maximum(0.0, 1.0 - r * r))) / bessel_i0(np.asarray(beta))


def kaiser_sinc_filter(cutoff, half_width, kernel_size):
    """2 fc w[n] sinc(2 fc t_n), normalized to unit sum; t_n is the
    half-integer grid n - K/2 + 1/2 for even K, the integer grid otherwise.
    Evaluated in float64 and returned as float32."""
    half_size = kernel_size // 2
    beta = kaiser_beta(cutoff, half_width, kernel_size)
    window = kaiser_window(kernel_size, beta)
    if kernel_size % 2 == 0:
        t = np.arange(kernel_size, dtype=F64) - half_size + 0.5
    else:
        t = np.arange(kernel_size, dtype=F64) - half_size
    x = 2.0 * cutoff * t
    sinc = np.where(x == 0.0, 1.0, np.sin(np.pi * x) / np.where(x == 0.0, 1.0, np.pi * x))
    filt = 2.0 * cutoff * window * sinc
    filt = filt / filt.sum()
    return filt.astype(F32)


# ---------------------------------------------------------------------------
# Weight norm (reading R2).
# ---------------------------------------------------------------------------

def fold_weight_norm(v, g):
    """w = g * v / ||v||, the norm taken over every axis of v except axis 0."""
    v64 = np.asarray(v, dtype=F64)
    g64 = np.asarray(g, dtype=F64).reshape((v64.shape[0],) + (1,) * (v64.ndim - 1))
    norm = np.sqrt(np.sum(v64 * v64, axis=tuple(range(1, v64.ndim)), keepdims=True))
    return _f32(g64 * v64 / norm)


# ---------------------------------------------------------------------------
# Convolutions (reading R1). x: (C_in, L) float32 for one batch item.
# ---------------------------------------------------------------------------

def conv1d(x, w, b=None, padding=0, dilation=1, stride=1):
    """y[o, t] = b[o] + sum_i sum_j w[o, i, j] x[i, t s + j d - p], with x = 0
    outside [0, L); output length floor((L + 2p - d (k - 1) - 1) / s) + 1."""
    x = np.asarray(x, dtype=F32)
    w = np.asarray(w, dtype=F32)
    c_out, c_in, k = w.shape
    assert x.shape[0] == c_in, (x.shape, w.shape)
    length = x.shape[1]
    l_out = (length + 2 * padding - dilation * (k - 1) - 1) // stride + 1
    assert l_out >= 1
    xp = np.zeros((c_in, length + 2 * padding), dtype=F64)
    xp[:, padding:padding + length] = x
    taps = np.ascontiguousarray(np.moveaxis(w.astype(F64), 2, 0))  # (k, C_out, C_in)
    y = np.zeros((c_out, l_out), dtype=F64)
    for j in range(k):
        y += taps[j] @ xp[:, j * dilation:j * dilation + stride * (l_out - 1) + 1:stride]
    if b is not None:
        y += np.asarray(b, dtype=F64)[:, None]
    return y.astype(F32)


def conv_transpose1d(x, w, b, stride, padding):
    """Transposed convolution: every input x[i, j] scatters w[i, o, q] x[i, j]
    into position j r + q - p; positions outside [0, (L-1) r - 2p + k) are
    dropped. w has shape (C_in, C_out, k)."""
    x = np.asarray(x, dtype=F32)
    w = np.asarray(w, dtype=F32)
    c_in, c_out, k = w.shape
    assert x.shape[0] == c_in
    length = x.shape[1]
    full_len = (length - 1) * stride + k
    full = np.zeros((c_out, full_len), dtype=F64)
    x64 = x.astype(F64)
    taps = np.ascontiguousarray(np.transpose(w.astype(F64), (2, 1, 0)))  # (k, C_out, C_in)
    for q in range(k):
        full[:, q:q + (length - 1) * stride + 1:stride] += taps[q] @ x64
    l_out = full_len - 2 * padding
    y = full[:, padding:padding + l_out]
    if b is not None:
        y = y + np.asarray(b, dtype=F64)[:, None]
    return y.astype(F32)


# ---------------------------------------------------------------------------
# Anti-aliased SnakeBeta (readings R4, R5). All arrays are (C, L), float64
# inside.
# ---------------------------------------------------------------------------

def upsample2(x, f):
    """Replicate-pad 5 on each side, transposed conv with stride 2 and the
    12-tap filter (zero insertion followed by the FIR), gain 2, crop 15 on
    each side: length L -> 2L."""
    x = np.asarray(x, dtype=F64)
    f = np.asarray(f, dtype=F64)
    k = f.shape[0]
    ratio = 2
    pad = k // ratio - 1
    crop_left = pad * ratio + (k - ratio) // 2
    crop_right = pad * ratio + (k - ratio + 1) // 2
    xp = np.pad(x, ((0, 0), (pad, pad)), mode="edge")
    n = xp.shape[1]
    full = np.zeros((x.shape[0], (n - 1) * ratio + k), dtype=F64)
    for q in range(k):
        full[:, q:q + (n - 1) * ratio + 1:ratio] += f[q] * xp
    return ratio * full[:, crop_left:full.shape[1] - crop_right]


def snake_beta(u, alpha, beta):
    """u + sin^2(alpha u) / beta, per channel."""
    a = np.asarray(alpha, dtype=F64).reshape(-1, 1)
    b = np.asarray(beta, dtype=F64).reshape(-1, 1)
    return u + np.sin(a * u) ** 2 / b


def downsample2(s, f):
    """Replicate-pad K/2 - 1 left and K/2 right, then the 12-tap FIR as a
    cross-correlation with stride 2: length 2L -> L."""
    s = np.asarray(s, dtype=F64)
    f = np.asarray(f, dtype=F64)
    k = f.shape[0]
    pad_left = k // 2 - (1 if k % 2 == 0 else 0)
    pad_right = k // 2
    sp = np.pad(s, ((0, 0), (pad_left, pad_right)), mode="edge")
    l_out = (sp.shape[1] - k) // 2 + 1
    y = np.zeros((s.shape[0], l_out), dtype=F64)
    for q in range(k):
        y += f[q] * sp[:, q:q + 2 * (l_out - 1) + 1:2]
    return y


def activation1d(x, alpha, beta, f_up, f_down):
    """Anti-aliased SnakeBeta: upsample2 -> SnakeBeta -> downsample2; the
    three steps in float64, the result rounded to float32 once."""
    u = upsample2(np.asarray(x, dtype=F32), f_up)
    s = snake_beta(u, alpha, beta)
    return downsample2(s, f_down).astype(F32)


# ---------------------------------------------------------------------------
# Parameter access.
# ---------------------------------------------------------------------------

def _conv_weight(params, prefix):
    """A conv's weight: folded from weight_v / weight_g, or taken as given
    when the parameter set holds an already-folded ``weight``."""
    if prefix + ".weight_v" in params:
        return fold_weight_norm(params[prefix + ".weight_v"], params[prefix + ".weight_g"])
    return np.asarray(params[prefix + ".weight"], dtype=F32)


def _act_params(params, prefix, default_filter):
    alpha = params[prefix + ".act.alpha"]
    beta = params[prefix + ".act.beta"]
    f_up = params.get(prefix + ".upsample.filter", default_filter)
    f_down = params.get(prefix + ".downsample.lowpass.filter", default_filter)
    return (np.asarray(alpha, dtype=F32).reshape(-1), np.asarray(beta, dtype=F32).reshape(-1),
            np.asarray(f_up, dtype=F32).reshape(-1), np.asarray(f_down, dtype=F32).reshape(-1))


def amp_block(x, params, prefix, kernel, dilations, default_filter):
    """Reading R3: for each dilation d, x <- x + conv2(act2(conv1(act1(x))))
    with conv1 of dilation d and conv2 of dilation 1, both "same"-padded."""
    for n, d in enumerate(dilations):
        a1 = _act_params(params, f"{prefix}.activations.{2 * n}", default_filter)
        a2 = _act_params(params, f"{prefix}.activations.{2 * n + 1}", default_filter)
        t = activation1d(x, *a1)
        t = conv1d(t, _conv_weight(params, f"{prefix}.convs1.{n}"), params[f"{prefix}.convs1.{n}.bias"],
                   padding=d * (kernel - 1) // 2, dilation=d)
        t = activation1d(t, *a2)
        t = conv1d(t, _conv_weight(params, f"{prefix}.convs2.{n}"), params[f"{prefix}.convs2.{n}.bias"],
                   padding=(kernel - 1) // 2, dilation=1)
        x = _f32(x.astype(F64) + t.astype(F64))
    return x


def stage_amp(h, params, stage, config=None, filt=None):
    """One stage's AMP set: the parallel blocks run from the same input and
    their outputs are averaged (``decode``: residual_sum / num_resblocks)."""
    cfg = dict(DEFAULT_CONFIG, **(config or {}))
    if filt is None:
        filt = kaiser_sinc_filter(cfg["filter_cutoff"], cfg["filter_half_width"], cfg["filter_taps"])
    kernels = cfg["resblock_kernel_sizes"]
    if len(kernels) == 0:
        raise RuntimeError("decoder has no residual blocks")
    acc = np.zeros(h.shape, dtype=F64)
    for j, k in enumerate(kernels):
        out = amp_block(h, params, f"decoder.resblocks.{stage * len(kernels) + j}", k,
                        cfg["resblock_dilation_sizes"][j], filt)
        acc += out.astype(F64)
    return _f32(acc / len(kernels))


def decode_item(params, z, config=None, denormalize=False, latents_mean=None, latents_std=None,
                clamp=True, return_stages=False):
    """One batch item: z (latent_channels, N) float32 -> (1, 800 N) float32.

    Follows ``MLXMiniMaxH3AudioVAE.decode``: dec_in_proj (1x1), conv_pre
    (pad 3), per upsampling stage a transposed conv with stride r and padding
    (k - r) // 2 followed by the averaged AMP blocks, then activation_post,
    conv_post (pad 3) and the clamp."""
    cfg = dict(DEFAULT_CONFIG, **(config or {}))
    filt = kaiser_sinc_filter(cfg["filter_cutoff"], cfg["filter_half_width"], cfg["filter_taps"])
    stages = []
    z = np.asarray(z, dtype=F32)
    if denormalize:
        mean = np.zeros(z.shape[0]) if latents_mean is None else np.asarray(latents_mean, dtype=F32)
        std = np.ones(z.shape[0]) if latents_std is None else np.asarray(latents_std, dtype=F32)
        z = _f32(z.astype(F64) * std.astype(F64)[:, None] + mean.astype(F64)[:, None])
    h = conv1d(z, params["dec_in_proj.weight"], params["dec_in_proj.bias"])
    stages.append(h)
    h = conv1d(h, _conv_weight(params, "decoder.conv_pre"), params["decoder.conv_pre.bias"], padding=3)
    stages.append(h)
    for s, (rate, kernel) in enumerate(zip(cfg["decoder_rates"], cfg["decoder_kernel_sizes"])):
        h = conv_transpose1d(h, _conv_weight(params, f"decoder.ups.{s}.0"), params[f"decoder.ups.{s}.0.bias"],
                             stride=rate, padding=(kernel - rate) // 2)
        stages.append(h)
        h = stage_amp(h, params, s, cfg, filt)
        stages.append(h)
    h = activation1d(h, *_act_params(params, "decoder.activation_post", filt))
    y = conv1d(h, _conv_weight(params, "decoder.conv_post"), params.get("decoder.conv_post.bias"), padding=3)
    if clamp:
        y = np.minimum(np.maximum(y, F32(-1.0)), F32(1.0))
    if return_stages:
        return y, stages
    return y


def decode(params, z, config=None, denormalize=False, latents_mean=None, latents_std=None, clamp=True):
    """Latents (B, latent_channels, N) -> waveform (B, 1, 800 N). Batch items
    (the stereo channels) decode independently and in order."""
    z = np.asarray(z, dtype=F32)
    assert z.ndim == 3
    return np.stack([decode_item(params, z[b], config, denormalize, latents_mean, latents_std, clamp)
                     for b in range(z.shape[0])])


def receptive_radius_latents(config=None):
    """Upper bound, in latents, on how far an output sample's dependence
    reaches into the latent sequence: the sum of every layer's one-sided
    reach converted to the latent rate (used to decode windows whose
    interior equals the full decode)."""
    cfg = dict(DEFAULT_CONFIG, **(config or {}))
    act_reach = 5  # a[n] reads x[n-5 .. n+5] (R4)
    reach = 0.0
    reach += 3  # conv_pre, k = 7, latent rate
    rate = 1
    for r, k in zip(cfg["decoder_rates"], cfg["decoder_kernel_sizes"]):
        reach += math.ceil(k / r) / rate  # transposed conv, input rate
        rate *= r
        block = 0
        for kk, dils in zip(cfg["resblock_kernel_sizes"], cfg["resblock_dilation_sizes"]):
            block = max(block, sum(d * (kk - 1) // 2 + (kk - 1) // 2 + 2 * act_reach for d in dils))
        reach += block / rate
    reach += (act_reach + 3) / rate  # activation_post + conv_post
    return reach


def decode_window(params, z, n0, n1, margin=None, config=None, denormalize=False, latents_mean=None,
                  latents_std=None, clamp=True):
    """Output samples [800 n0, 800 n1) of the full decode of z (B, C, N),
    computed from the latent window [n0 - margin, n1 + margin) cut to the
    sequence; the margin exceeds the receptive radius, so the cropped
    result equals the full decode's samples."""
    cfg = dict(DEFAULT_CONFIG, **(config or {}))
    hop = int(np.prod(cfg["decoder_rates"]))
    if margin is None:
        margin = int(math.ceil(receptive_radius_latents(cfg))) + 1
    n_total = z.shape[2]
    a = max(0, n0 - margin)
    b = min(n_total, n1 + margin)
    y = decode(params, z[:, :, a:b], cfg, denormalize, latents_mean, latents_std, clamp)
    return y[:, :, (n0 - a) * hop:(n1 - a) * hop]


# ---------------------------------------------------------------------------
# Encoder convolution stack (FastVideo "minimax_h3_audio_vae", source of
# ``MLXMiniMaxH3AudioVAE.encode`` up to ``hidden``; readings E1-E3)
# ---------------------------------------------------------------------------

def snake(x, alpha):
    """Plain Snake (reading E1): x + sin^2(alpha x) / (alpha + 1e-9), alpha
    per channel of x (C, L)."""
    x64 = np.asarray(x, dtype=F64)
    a = np.asarray(alpha, dtype=F64).reshape(-1)[:, None]
    return _f32(x64 + np.sin(a * x64) ** 2 / (a + 1e-9))


def _enc_conv(params, prefix):
    w = fold_weight_norm(params[prefix + ".weight_v"], params[prefix + ".weight_g"])
    return w, params[prefix + ".bias"]


def encode_hidden_item(params, wave, config=None):
    """One waveform (S,) -> hidden (latent_dim, ceil(S / hop)): right zero
    pad to a whole number of hops, k7 conv, then per stride s a block of
    three plain-Snake residual units (dilations 1, 3, 9: snake, k7 dilated
    conv, snake, k1 conv, add) followed by snake and a conv of kernel 2s,
    stride s, padding ceil(s / 2) that doubles the width; last a snake and
    a k3 conv."""
    cfg = dict(DEFAULT_CONFIG, **(config or {}))
    hop = int(np.prod(cfg["encoder_rates"]))
    x = np.asarray(wave, dtype=F32).reshape(1, -1)
    samples = x.shape[1]
    right_pad = -(-samples // hop) * hop - samples
    if right_pad:
        x = np.concatenate([x, np.zeros((1, right_pad), dtype=F32)], axis=1)
    w, b = _enc_conv(params, "encoder.block.0")
    x = conv1d(x, w, b, padding=3)
    for index, stride in enumerate(cfg["encoder_rates"], start=1):
        prefix = f"encoder.block.{index}"
        for unit, dilation in enumerate((1, 3, 9)):
            p = f"{prefix}.block.{unit}"
            r = snake(x, params[p + ".block.0.alpha"])
            w, b = _enc_conv(params, p + ".block.1")
            r = conv1d(r, w, b, padding=(7 - 1) * dilation // 2, dilation=dilation)
            r = snake(r, params[p + ".block.2.alpha"])
            w, b = _enc_conv(params, p + ".block.3")
            r = conv1d(r, w, b)
            assert r.shape == x.shape  # reading E3: no crop
            x = _f32(x.astype(F64) + r.astype(F64))
        x = snake(x, params[prefix + ".block.3.alpha"])
        w, b = _enc_conv(params, prefix + ".block.4")
        length = x.shape[1]
        x = conv1d(x, w, b, stride=stride, padding=-(-stride // 2))
        assert x.shape[1] * stride == length
    n = len(cfg["encoder_rates"])
    x = snake(x, params[f"encoder.block.{n + 1}.alpha"])
    w, b = _enc_conv(params, f"encoder.block.{n + 2}")
    return conv1d(x, w, b, padding=1)


def encode_hidden(params, wave, config=None):
    """Waveforms (B, 1, S) -> hidden (B, latent_dim, ceil(S / hop))."""
    wave = np.asarray(wave, dtype=F32)
    return np.stack([encode_hidden_item(params, wave[i].reshape(-1), config) for i in range(wave.shape[0])])


# ---------------------------------------------------------------------------
# Attention projection ``pre_block`` and the posterior mean (FastVideo
# "minimax_h3_audio_vae", module overview, Encoder bullet, and the source of
# ``encode``; diffusers "AutoencoderKLMiniMaxH3Audio", introduction and
# section "encode"; readings P1-P8)
# ---------------------------------------------------------------------------

def gelu(x):
    """Exact GELU: x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, in float64."""
    x = np.asarray(x, dtype=F64)
    erf = np.frompyfunc(math.erf, 1, 1)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)).astype(F64))


def qkv_bias(params, dim):
    """(b_q, 0, b_v) of length 3D (reading P1): separate q / v biases, or the
    q and v thirds of a fused bias; the k third is zero either way."""
    if "pre_block.attn.q_bias" in params:
        bq = np.asarray(params["pre_block.attn.q_bias"], dtype=F64).reshape(-1)
        bv = np.asarray(params["pre_block.attn.v_bias"], dtype=F64).reshape(-1)
    elif "pre_block.attn.qkv.bias" in params:
        b = np.asarray(params["pre_block.attn.qkv.bias"], dtype=F64).reshape(-1)
        bq, bv = b[:dim], b[2 * dim:]
    else:
        bq = bv = np.zeros(dim)
    return np.concatenate([bq, np.zeros(dim), bv])


def causal_attention_heads_mean(q, k, v, heads):
    """q, k, v (N, D) float32 -> (N, D / heads): per head h (features
    [h hd, (h + 1) hd)), softmax over u <= t of q_t . k_u / sqrt(hd),
    times v_u, then the mean over the heads (readings P2, P3). float64
    inside, float32 out."""
    q, k, v = (np.asarray(a, dtype=F64) for a in (q, k, v))
    n, dim = q.shape
    hd = dim // heads
    future = np.triu(np.ones((n, n), dtype=bool), 1)
    out = np.zeros((n, hd), dtype=F64)
    for h in range(heads):
        sl = slice(h * hd, (h + 1) * hd)
        s = q[:, sl] @ k[:, sl].T / math.sqrt(hd)
        s[future] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out += p @ v[:, sl]
    return _f32(out / heads)


def pre_block_item(params, hidden, config=None):
    """The attention projection of one item: hidden (D, N) float32 ->
    (C, N) float32, C = latent_channels (readings P1-P7)."""
    cfg = dict(DEFAULT_CONFIG, **(config or {}))
    heads, c = cfg["num_attention_heads"], cfg["latent_channels"]
    x = np.asarray(hidden, dtype=F32).T  # tokens = frames
    dim = x.shape[1]
    hd = dim // heads
    assert hd * heads == dim and hd % c == 0, (dim, heads, c)
    w = np.asarray(params["pre_block.attn.qkv.weight"], dtype=F64)
    qkv = _f32(x.astype(F64) @ w.T + qkv_bias(params, dim))
    o = causal_attention_heads_mean(qkv[:, :dim], qkv[:, dim:2 * dim], qkv[:, 2 * dim:], heads)
    a = _f32(o.astype(F64).reshape(o.shape[0], c, hd // c).mean(axis=2))

    def linear(z, name):
        return z.astype(F64) @ np.asarray(params[name + ".weight"], dtype=F64).T + \
            np.asarray(params[name + ".bias"], dtype=F64)

    y = _f32(linear(a, "pre_block.attn.proj"))
    hcat = linear(y, "pre_block.mlp.fc1")
    f = hcat.shape[1] // 2
    m = _f32(hcat[:, :f] * gelu(hcat[:, f:]))
    return _f32(linear(m, "pre_block.mlp.fc2")).T


def encode_item(params, wave, config=None):
    """One waveform (S,) -> the posterior mean (latent_channels, ceil(S / hop)):
    the convolution stack, the attention projection, then mean_proj (1x1
    conv with bias)."""
    hidden = encode_hidden_item(params, wave, config)
    proj = pre_block_item(params, hidden, config)
    return conv1d(proj, params["mean_proj.weight"], params["mean_proj.bias"])


def encode(params, wave, config=None):
    """Waveforms (B, 1, S) -> posterior means (B, latent_channels, ceil(S / hop));
    items are independent."""
    wave = np.asarray(wave, dtype=F32)
    return np.stack([encode_item(params, wave[i].reshape(-1), config) for i in range(wave.shape[0])])
