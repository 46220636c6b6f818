"""Pins of the CPU oracle to facts that do not come from the oracle itself:
library routines that implement the same textbook operation (scipy's Kaiser
design, torch's convolutions and weight norm), closed forms derived by hand
from the definitions, brute-force sums on tiny inputs, and invariants of the
method (DC gain, impulse response, length laws, batch independence,
linearity, shift equivariance)."""

import math

import numpy as np
import pytest
import scipy.signal as ss
import scipy.special as sp
import torch
import torch.nn.functional as F

import oracle as O
from neural_audio_vae_amd import synth
from tests.conftest import SMALL_CONFIG

F64 = torch.float64


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------------------
# Kaiser-windowed sinc low-pass (FastVideo "minimax_h3_audio_vae",
# kaiser_sinc_filter1d)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("x", [0.0, 0.1, 1.0, 2.5, 4.6638, 10.0, 30.0])
def test_bessel_i0_matches_scipy(x):
    assert O.bessel_i0(x) == pytest.approx(sp.i0(x), rel=1e-14)


@pytest.mark.parametrize("ksize,hw", [(12, 0.3), (6, 0.3), (4, 0.1), (16, 0.2), (11, 0.3)])
def test_kaiser_beta_matches_scipy_design_rules(ksize, hw):
    # The page's attenuation is scipy's kaiser_atten with (half_size - 1)
    # in place of (numtaps - 1), i.e. numtaps = half_size, and width 4 hw;
    # its three-branch beta is scipy's kaiser_beta.
    atten = ss.kaiser_atten(ksize // 2, 4 * hw)
    assert O.kaiser_beta(0.25, hw, ksize) == pytest.approx(ss.kaiser_beta(atten), rel=1e-13, abs=1e-15)


def test_kaiser_beta_default_value():
    # 2.285 * 5 * pi * 1.2 + 7.95 = 51.0212... > 50, beta = 0.1102 (A - 8.7)
    atten = 2.285 * 5 * math.pi * 1.2 + 7.95
    assert atten > 50
    assert O.kaiser_beta(0.25, 0.3, 12) == pytest.approx(4.66380013, abs=1e-8)


@pytest.mark.parametrize("n,beta", [(12, 4.6638), (11, 3.0), (2, 1.0), (31, 8.0)])
def test_kaiser_window_matches_scipy(n, beta):
    np.testing.assert_allclose(O.kaiser_window(n, beta), ss.windows.kaiser(n, beta, sym=True), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("ksize,cutoff,hw", [(12, 0.25, 0.3), (11, 0.25, 0.3), (16, 0.2, 0.25), (12, 0.1, 0.3)])
def test_filter_matches_scipy_firwin(ksize, cutoff, hw):
    # firwin builds the same windowed sinc on the grid n - (K-1)/2 (half
    # integers for even K, integers for odd K) with the cutoff as a fraction
    # of Nyquist (2 fc), and scales it to unit DC gain.
    beta = O.kaiser_beta(cutoff, hw, ksize)
    ref = ss.firwin(ksize, 2 * cutoff, window=("kaiser", beta), scale=True)
    got = O.kaiser_sinc_filter(cutoff, hw, ksize).astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-8)


def test_filter_properties():
    f = O.kaiser_sinc_filter(0.25, 0.3, 12).astype(np.float64)
    assert f.dtype == np.float64 and f.shape == (12,)
    assert abs(f.sum() - 1.0) < 1e-7
    np.testing.assert_array_equal(f, f[::-1])
    # Symmetry of a 12-tap filter maps even taps onto odd ones, so each
    # polyphase branch sums to one half.
    assert abs(f[0::2].sum() - 0.5) < 1e-7 and abs(f[1::2].sum() - 0.5) < 1e-7
    # Centre taps dominate, outermost taps are small and positive.
    assert f[5] > 0.4 and 0 < f[0] < 0.01


# ---------------------------------------------------------------------------
# Weight norm (reading: norm over all axes but axis 0)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(6, 4, 3), (4, 6, 9), (1, 8, 7)])
def test_weight_norm_matches_torch(shape):
    rng = np.random.default_rng(1)
    v = rng.standard_normal(shape).astype(np.float32)
    g = rng.uniform(0.5, 1.5, size=(shape[0], 1, 1)).astype(np.float32)
    ref = torch._weight_norm(torch.tensor(v, dtype=F64), torch.tensor(g, dtype=F64), 0).numpy()
    np.testing.assert_allclose(O.fold_weight_norm(v, g), ref, rtol=1e-6, atol=0)


def test_weight_norm_invariants():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((5, 3, 4)).astype(np.float32)
    norm = np.sqrt((v.astype(np.float64) ** 2).sum(axis=(1, 2)))
    np.testing.assert_allclose(O.fold_weight_norm(v, norm.reshape(5, 1, 1)), v, rtol=2e-7)
    g = rng.uniform(0.5, 2, size=(5, 1, 1)).astype(np.float32)
    np.testing.assert_allclose(O.fold_weight_norm(3.5 * v, g), O.fold_weight_norm(v, g), rtol=2e-7)
    w = O.fold_weight_norm(v, -g).astype(np.float64)
    np.testing.assert_allclose(np.sqrt((w ** 2).sum(axis=(1, 2))), g.reshape(-1), rtol=1e-6)


# ---------------------------------------------------------------------------
# Convolutions: brute-force double sums on tiny shapes, and torch
# ---------------------------------------------------------------------------

def brute_conv1d(x, w, b, p, d):
    """Scatter form: every input sample x[i, s] adds w[o, i, j] x[i, s] to
    the output t with t + j d - p = s."""
    c_out, c_in, k = w.shape
    length = x.shape[1]
    l_out = length + 2 * p - d * (k - 1)
    y = [[float(b[o]) for _ in range(l_out)] for o in range(c_out)]
    for o in range(c_out):
        for i in range(c_in):
            for j in range(k):
                for s in range(length):
                    t = s - j * d + p
                    if 0 <= t < l_out:
                        y[o][t] += float(w[o, i, j]) * float(x[i, s])
    return np.array(y)


def brute_conv_transpose1d(x, w, b, r, p):
    """Gather form: y[o, t] = b[o] + sum over (i, j, q) with j r + q - p = t."""
    c_in, c_out, k = w.shape
    length = x.shape[1]
    l_out = (length - 1) * r - 2 * p + k
    y = np.zeros((c_out, l_out))
    for o in range(c_out):
        for t in range(l_out):
            acc = float(b[o])
            for i in range(c_in):
                for j in range(length):
                    q = t + p - j * r
                    if 0 <= q < k:
                        acc += float(w[i, o, q]) * float(x[i, j])
            y[o, t] = acc
    return y


@pytest.mark.parametrize("k,d", [(1, 1), (3, 1), (3, 5), (7, 1), (7, 3), (11, 1), (11, 5), (4, 2)])
def test_conv1d_matches_brute_force(k, d):
    rng = np.random.default_rng(10 * k + d)
    c_in, c_out, length = 3, 4, 9
    p = d * (k - 1) // 2
    if length + 2 * p - d * (k - 1) < 1:
        pytest.skip("empty output")
    x = rng.standard_normal((c_in, length)).astype(np.float32)
    w = rng.standard_normal((c_out, c_in, k)).astype(np.float32)
    b = rng.standard_normal(c_out).astype(np.float32)
    got = O.conv1d(x, w, b, padding=p, dilation=d).astype(np.float64)
    ref = brute_conv1d(x, w, b, p, d)
    assert got.shape == ref.shape == (c_out, length + 2 * p - d * (k - 1))
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("k,d,p", [(3, 1, 1), (7, 3, 9), (11, 5, 25), (7, 1, 3), (1, 1, 0), (5, 2, 0)])
def test_conv1d_matches_torch(k, d, p):
    rng = np.random.default_rng(k * 100 + d)
    x = rng.standard_normal((2, 6, 40)).astype(np.float32)
    w = rng.standard_normal((5, 6, k)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    ref = F.conv1d(torch.tensor(x, dtype=F64), torch.tensor(w, dtype=F64), torch.tensor(b, dtype=F64),
                   padding=p, dilation=d).numpy()
    for bi in range(2):
        np.testing.assert_allclose(O.conv1d(x[bi], w, b, padding=p, dilation=d), ref[bi], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("r,k", [(5, 9), (2, 4), (3, 7), (4, 4)])
def test_conv_transpose1d_matches_brute_force(r, k):
    rng = np.random.default_rng(r * 31 + k)
    c_in, c_out, length = 3, 2, 6
    p = (k - r) // 2
    x = rng.standard_normal((c_in, length)).astype(np.float32)
    w = rng.standard_normal((c_in, c_out, k)).astype(np.float32)
    b = rng.standard_normal(c_out).astype(np.float32)
    got = O.conv_transpose1d(x, w, b, r, p).astype(np.float64)
    ref = brute_conv_transpose1d(x, w, b, r, p)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("r,k", [(5, 9), (2, 4)])
def test_conv_transpose1d_matches_torch(r, k):
    rng = np.random.default_rng(r + 7 * k)
    x = rng.standard_normal((8, 33)).astype(np.float32)
    w = rng.standard_normal((8, 5, k)).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    p = (k - r) // 2
    ref = F.conv_transpose1d(torch.tensor(x[None], dtype=F64), torch.tensor(w, dtype=F64),
                             torch.tensor(b, dtype=F64), stride=r, padding=p).numpy()[0]
    np.testing.assert_allclose(O.conv_transpose1d(x, w, b, r, p), ref, rtol=1e-6, atol=1e-6)


def test_transposed_conv_length_law():
    # (L - 1) r - 2p + k = r L with p = (k - r) // 2 for every stage.
    x = np.ones((1, 7), dtype=np.float32)
    for r, k in zip(O.DEFAULT_CONFIG["decoder_rates"], O.DEFAULT_CONFIG["decoder_kernel_sizes"]):
        w = np.ones((1, 1, k), dtype=np.float32)
        assert O.conv_transpose1d(x, w, None, r, (k - r) // 2).shape == (1, 7 * r)
    assert int(np.prod(O.DEFAULT_CONFIG["decoder_rates"])) == O.DEFAULT_CONFIG["hop_length"] == 800


# ---------------------------------------------------------------------------
# Anti-aliased activation: up 2x -> SnakeBeta -> down 2x
# ---------------------------------------------------------------------------

FILT = O.kaiser_sinc_filter(0.25, 0.3, 12)


def torch_upsample2(x, f):
    """Replicate pad 5, grouped transposed conv (stride 2), gain 2, crop 15/15
    -- the same operation composed from torch library routines."""
    c = x.shape[0]
    xt = F.pad(torch.tensor(x[None], dtype=F64), (5, 5), mode="replicate")
    ft = torch.tensor(f, dtype=F64).view(1, 1, -1).expand(c, 1, 12).contiguous()
    return (2 * F.conv_transpose1d(xt, ft, stride=2, groups=c))[0, :, 15:-15].numpy()


def torch_downsample2(s, f):
    c = s.shape[0]
    st = F.pad(torch.tensor(s[None], dtype=F64), (5, 6), mode="replicate")
    ft = torch.tensor(f, dtype=F64).view(1, 1, -1).expand(c, 1, 12).contiguous()
    return F.conv1d(st, ft, stride=2, groups=c)[0].numpy()


def brute_upsample2(x, f):
    """Polyphase form derived by hand: with X the replicate-extended input,
    u[2t] = 2 sum_{e=-2..3} X[t-e] f[5+2e] and
    u[2t+1] = 2 sum_{e=-3..2} X[t-e] f[6+2e]."""
    c, length = x.shape
    u = np.zeros((c, 2 * length))
    for ch in range(c):
        X = lambda m: float(x[ch, min(max(m, 0), length - 1)])  # noqa: E731
        for t in range(length):
            u[ch, 2 * t] = 2 * sum(X(t - e) * float(f[5 + 2 * e]) for e in range(-2, 4))
            u[ch, 2 * t + 1] = 2 * sum(X(t - e) * float(f[6 + 2 * e]) for e in range(-3, 3))
    return u


def brute_downsample2(s, f):
    """a[n] = sum_q f[q] s[clamp(2n + q - 5)]."""
    c, n2 = s.shape
    out = np.zeros((c, n2 // 2))
    for ch in range(c):
        for n in range(n2 // 2):
            out[ch, n] = sum(float(f[q]) * float(s[ch, min(max(2 * n + q - 5, 0), n2 - 1)]) for q in range(12))
    return out


@pytest.mark.parametrize("length", [1, 2, 5, 11, 40])
def test_upsample_matches_torch_and_polyphase(length):
    x = np.random.default_rng(length).standard_normal((3, length)).astype(np.float32)
    got = O.upsample2(x, FILT)
    assert got.shape == (3, 2 * length)
    np.testing.assert_allclose(got, torch_upsample2(x, FILT), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, brute_upsample2(x, FILT), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("length", [1, 2, 5, 11, 40])
def test_downsample_matches_torch_and_brute(length):
    s = np.random.default_rng(100 + length).standard_normal((3, 2 * length))
    got = O.downsample2(s, FILT)
    assert got.shape == (3, length)
    np.testing.assert_allclose(got, torch_downsample2(s, FILT), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, brute_downsample2(s, FILT), rtol=1e-12, atol=1e-12)


def test_resampler_dc_gain():
    # A constant passes the upsampler and the up->down cascade unchanged:
    # each polyphase branch sums to 1/2 and the gain is 2.
    c = np.full((2, 17), 0.7311, dtype=np.float32)
    np.testing.assert_allclose(O.upsample2(c, FILT), 0.7311, rtol=1e-7)
    np.testing.assert_allclose(O.downsample2(O.upsample2(c, FILT), FILT), 0.7311, rtol=1e-7)


def test_resampler_impulse_response_is_even_autocorrelation():
    # With an identity activation, up->down is LTI with impulse response
    # h[m] = 2 (f * f)[2m] (f symmetric, so autocorrelation = convolution),
    # centred on the impulse: zero delay, gain 2 on the even lags.
    n0, length = 30, 61
    x = np.zeros((1, length), dtype=np.float32)
    x[0, n0] = 1.0
    y = O.downsample2(O.upsample2(x, FILT), FILT)[0]
    ac = np.correlate(FILT.astype(np.float64), FILT.astype(np.float64), mode="full")  # lags -11..11
    h = 2 * ac[1::2]  # even lags -10..10 -> m = -5..5
    expect = np.zeros(length)
    expect[n0 - 5:n0 + 6] = h
    np.testing.assert_allclose(y, expect, atol=1e-12)


def test_resampler_passes_low_frequency_sine_without_delay():
    n = np.arange(400)
    x = np.sin(2 * np.pi * 0.02 * n)[None].astype(np.float32)
    y = O.downsample2(O.upsample2(x, FILT), FILT)[0]
    inner = slice(20, 380)
    assert np.max(np.abs(y[inner] - x[0, inner])) < 5e-4


def test_snake_beta_closed_forms():
    u = np.array([[0.0, 0.3, -2.0, math.pi / 2]])
    np.testing.assert_allclose(O.snake_beta(u, [1e-30], [0.7]), u, atol=1e-15)
    # alpha u = pi/2 -> u + 1/beta
    np.testing.assert_allclose(O.snake_beta(np.array([[math.pi / 2]]), [1.0], [0.8]), math.pi / 2 + 1.25)
    # sin^2 is even in u
    np.testing.assert_allclose(O.snake_beta(np.array([[1.3]]), [1.1], [0.6]) - 1.3,
                               O.snake_beta(np.array([[-1.3]]), [1.1], [0.6]) + 1.3)


def test_activation_alpha_to_zero_is_resampler_only():
    x = np.random.default_rng(5).standard_normal((2, 50)).astype(np.float32)
    got = O.activation1d(x, [0.0, 0.0], [1.0, 1.0], FILT, FILT)
    ref = torch_downsample2(torch_upsample2(x, FILT), FILT)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


def test_activation_of_constant():
    c = 0.9
    x = np.full((1, 23), c, dtype=np.float32)
    got = O.activation1d(x, [1.3], [0.7], FILT, FILT)
    c32 = float(np.float32(c))
    np.testing.assert_allclose(got, c32 + math.sin(1.3 * c32) ** 2 / 0.7, rtol=1e-6)


# ---------------------------------------------------------------------------
# Whole decoder: structure and invariants
# ---------------------------------------------------------------------------

def zero_alpha_bias(params):
    p = dict(params)
    for name in p:
        if name.endswith(".alpha") or name.endswith(".bias"):
            p[name] = np.zeros_like(p[name])
    return p


def test_clamp_keeps_nan_as_torch_clamp(small_params):
    # The decode's final clamp follows torch.clamp (the pages' module) on
    # non-finite values: NaN stays NaN, +-inf saturate. A NaN latent spreads
    # only within the receptive radius (about 31 latents), so late samples
    # stay finite.
    v = np.array([np.nan, 2.0, -3.0, np.inf, -np.inf, 0.25], np.float32)
    want = torch.clamp(torch.from_numpy(v), -1.0, 1.0).numpy()
    got = np.minimum(np.maximum(v, np.float32(-1.0)), np.float32(1.0))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_array_equal(got[~np.isnan(want)], want[~np.isnan(want)])
    z = synth.make_latents(1, 80, seed=11, channels=4)
    z[0, 2, 5] = np.nan
    y = O.decode(small_params, z, SMALL_CONFIG, clamp=True)[0, 0]
    u = O.decode(small_params, z, SMALL_CONFIG, clamp=False)[0, 0]
    np.testing.assert_array_equal(np.isnan(y), np.isnan(u))
    assert np.isnan(y[800 * 5]) and not np.isnan(y[800 * 60:]).any()
    fin = ~np.isnan(u)
    np.testing.assert_array_equal(y[fin], torch.clamp(torch.from_numpy(u[fin]), -1.0, 1.0).numpy())


@pytest.mark.parametrize("n", [1, 4])
def test_decode_length_and_clamp(default_params, n):
    z = synth.make_latents(1, n)
    y = O.decode(default_params, z)
    assert y.shape == (1, 1, 800 * n) and y.dtype == np.float32
    assert np.all(y <= 1.0) and np.all(y >= -1.0)
    assert np.all(np.isfinite(O.decode(default_params, z, clamp=False)))


def test_decode_batch_items_independent_and_in_order(small_params):
    z = synth.make_latents(2, 6, channels=4)
    both = O.decode(small_params, z, SMALL_CONFIG, clamp=False)
    np.testing.assert_array_equal(both[0], O.decode(small_params, z[:1], SMALL_CONFIG, clamp=False)[0])
    np.testing.assert_array_equal(both[1], O.decode(small_params, z[1:], SMALL_CONFIG, clamp=False)[0])
    assert not np.array_equal(both[0], both[1])


def test_decode_linear_when_snake_and_biases_vanish(small_params):
    p = zero_alpha_bias(small_params)
    z1 = synth.make_latents(1, 5, seed=1, channels=4)
    z2 = synth.make_latents(1, 5, seed=2, channels=4)
    a, b = 0.75, -1.5
    lhs = O.decode(p, a * z1 + b * z2, SMALL_CONFIG, clamp=False)
    rhs = a * O.decode(p, z1, SMALL_CONFIG, clamp=False).astype(np.float64) + \
        b * O.decode(p, z2, SMALL_CONFIG, clamp=False).astype(np.float64)
    assert rel_l2(lhs, rhs) < 1e-5


def test_decode_shift_equivariant_in_the_interior(small_params):
    # Every layer is a finite stencil, so dropping s leading latents shifts
    # the output by 800 s, away from both ends of the sequence.
    n, s = 90, 3
    z = synth.make_latents(1, n, seed=4, channels=4)
    full = O.decode(small_params, z, SMALL_CONFIG, clamp=False)[0, 0]
    cut = O.decode(small_params, z[:, :, s:], SMALL_CONFIG, clamp=False)[0, 0]
    margin = int(math.ceil(O.receptive_radius_latents())) * 800
    lo, hi = margin, (n - s) * 800 - margin
    assert hi - lo > 800 * 20
    np.testing.assert_allclose(cut[lo:hi], full[lo + 800 * s:hi + 800 * s], rtol=1e-6, atol=1e-6)
    # ... while near the left end the replicate / zero padding makes them differ.
    assert np.max(np.abs(cut[:800] - full[800 * s:800 * s + 800])) > 1e-3


def test_receptive_radius_bounds_dependence(small_params):
    # Perturbing a latent just outside the derived radius leaves a sample
    # untouched; one well inside it changes the sample.
    n = 80
    radius = int(math.ceil(O.receptive_radius_latents()))
    z = synth.make_latents(1, n, seed=6, channels=4)
    base = O.decode(small_params, z, SMALL_CONFIG, clamp=False)[0, 0]
    t = 10 * 800 + 400  # an output sample inside latent 10
    far = z.copy()
    far[0, :, 10 + radius + 1] += 3.0
    near = z.copy()
    near[0, :, 12] += 3.0
    assert O.decode(small_params, far, SMALL_CONFIG, clamp=False)[0, 0, t] == base[t]
    assert O.decode(small_params, near, SMALL_CONFIG, clamp=False)[0, 0, t] != base[t]


def test_decode_window_equals_full_decode(small_params):
    z = synth.make_latents(2, 100, seed=7, channels=4)
    full = O.decode(small_params, z, SMALL_CONFIG, clamp=False)
    for n0, n1 in [(0, 3), (48, 52), (96, 100)]:
        win = O.decode_window(small_params, z, n0, n1, config=SMALL_CONFIG, clamp=False)
        np.testing.assert_allclose(win, full[:, :, 800 * n0:800 * n1], rtol=1e-6, atol=1e-6)


def test_decode_reduces_to_conv_chain_without_amp(small_params):
    # With every AMP conv weight and bias zeroed each block returns its
    # input, so a stage is its transposed conv; the decoder is then a chain
    # of textbook layers, composed here from torch library routines.
    p = dict(small_params)
    for name in p:
        if ".resblocks." in name and (".convs" in name) and (name.endswith(".bias") or name.endswith("_g")):
            p[name] = np.zeros_like(p[name])
    cfg = dict(O.DEFAULT_CONFIG, **SMALL_CONFIG)
    z = synth.make_latents(1, 3, seed=8, channels=4)
    got = O.decode(p, z, SMALL_CONFIG, clamp=False)[0]

    def T(a):
        return torch.tensor(np.asarray(a), dtype=F64)

    def wn(pref):
        return torch._weight_norm(T(p[pref + ".weight_v"]), T(p[pref + ".weight_g"]), 0)

    h = F.conv1d(T(z), T(p["dec_in_proj.weight"]), T(p["dec_in_proj.bias"]))
    h = F.conv1d(h, wn("decoder.conv_pre"), T(p["decoder.conv_pre.bias"]), padding=3)
    for s, (r, k) in enumerate(zip(cfg["decoder_rates"], cfg["decoder_kernel_sizes"])):
        h = F.conv_transpose1d(h, wn(f"decoder.ups.{s}.0"), T(p[f"decoder.ups.{s}.0.bias"]), stride=r,
                               padding=(k - r) // 2)
    c = h.shape[1]
    f = T(FILT).view(1, 1, -1).expand(c, 1, 12).contiguous()
    u = 2 * F.conv_transpose1d(F.pad(h, (5, 5), mode="replicate"), f, stride=2, groups=c)[..., 15:-15]
    a = T(p["decoder.activation_post.act.alpha"]).view(1, -1, 1)
    b = T(p["decoder.activation_post.act.beta"]).view(1, -1, 1)
    u = u + torch.sin(a * u) ** 2 / b
    h = F.conv1d(F.pad(u, (5, 6), mode="replicate"), f, stride=2, groups=c)
    ref = F.conv1d(h, wn("decoder.conv_post"), T(p["decoder.conv_post.bias"]), padding=3)[0].numpy()
    assert rel_l2(got, ref) < 1e-5


def test_denormalization_is_per_channel_affine(small_params):
    z = synth.make_latents(1, 4, seed=9, channels=4)
    mean = np.array([0.1, -0.2, 0.05, 0.0], dtype=np.float32)
    std = np.array([0.5, 2.0, 1.0, 1.5], dtype=np.float32)
    a = O.decode(small_params, z, SMALL_CONFIG, denormalize=True, latents_mean=mean, latents_std=std, clamp=False)
    zz = (z.astype(np.float64) * std[None, :, None] + mean[None, :, None]).astype(np.float32)
    np.testing.assert_array_equal(a, O.decode(small_params, zz, SMALL_CONFIG, clamp=False))


def test_zero_resblocks_rejected(small_params):
    with pytest.raises(RuntimeError):
        O.stage_amp(np.zeros((64, 5), dtype=np.float32), small_params, 0, dict(SMALL_CONFIG, resblock_kernel_sizes=()))


def torch_act(x, alpha, beta):
    c = x.shape[1]
    f = torch.tensor(FILT, dtype=F64).view(1, 1, -1).expand(c, 1, 12).contiguous()
    u = 2 * F.conv_transpose1d(F.pad(x, (5, 5), mode="replicate"), f, stride=2, groups=c)[..., 15:-15]
    u = u + torch.sin(alpha.view(1, -1, 1) * u) ** 2 / beta.view(1, -1, 1)
    return F.conv1d(F.pad(u, (5, 6), mode="replicate"), f, stride=2, groups=c)


@pytest.mark.parametrize("block", [0, 1, 2])
def test_amp_stage_matches_torch_composition(small_params, block):
    # The AMP set of stage 3 (8 channels in the narrow decoder) against the
    # same reading composed from torch's dilated conv1d and grouped
    # resampling convs: per dilation d, x + conv_{k,1}(act(conv_{k,d}(act(x)))).
    p = small_params
    stage = 3
    x = synth.make_signal((8, 37), seed=11)
    kernels = (3, 7, 11)

    def T(a):
        return torch.tensor(np.asarray(a), dtype=F64)

    outs = []
    for j, k in enumerate(kernels):
        pre = f"decoder.resblocks.{3 * stage + j}"
        h = T(x[None])
        for n, d in enumerate((1, 3, 5)):
            w1 = torch._weight_norm(T(p[f"{pre}.convs1.{n}.weight_v"]), T(p[f"{pre}.convs1.{n}.weight_g"]), 0)
            w2 = torch._weight_norm(T(p[f"{pre}.convs2.{n}.weight_v"]), T(p[f"{pre}.convs2.{n}.weight_g"]), 0)
            t = torch_act(h, T(p[f"{pre}.activations.{2 * n}.act.alpha"]), T(p[f"{pre}.activations.{2 * n}.act.beta"]))
            t = F.conv1d(t, w1, T(p[f"{pre}.convs1.{n}.bias"]), padding=d * (k - 1) // 2, dilation=d)
            t = torch_act(t, T(p[f"{pre}.activations.{2 * n + 1}.act.alpha"]),
                          T(p[f"{pre}.activations.{2 * n + 1}.act.beta"]))
            t = F.conv1d(t, w2, T(p[f"{pre}.convs2.{n}.bias"]), padding=(k - 1) // 2)
            h = h + t
        outs.append(h[0].numpy())
        if j == block:
            got = O.amp_block(x, p, pre, k, (1, 3, 5), FILT)
            assert rel_l2(got, outs[-1]) < 1e-6
    if block == 2:
        got = O.stage_amp(x, p, stage, SMALL_CONFIG)
        assert rel_l2(got, sum(outs) / 3) < 1e-6


# ---------------------------------------------------------------------------
# Encoder convolution stack (FastVideo "minimax_h3_audio_vae", source of
# MLXMiniMaxH3AudioVAE.encode up to `hidden`; readings E1-E3)
# ---------------------------------------------------------------------------

ENC_SMALL = {"encoder_dim": 4, "latent_dim": 16}


@pytest.mark.parametrize("k,s,p,d", [(4, 2, 1, 1), (8, 4, 2, 1), (10, 5, 3, 1), (7, 1, 9, 3), (3, 2, 0, 2)])
def test_conv1d_stride_matches_brute_force_and_torch(k, s, p, d):
    rng = np.random.default_rng(k * 10 + s)
    x = rng.standard_normal((3, 23)).astype(np.float32)
    w = rng.standard_normal((2, 3, k)).astype(np.float32)
    b = rng.standard_normal(2).astype(np.float32)
    got = O.conv1d(x, w, b, padding=p, dilation=d, stride=s)
    l_out = (23 + 2 * p - d * (k - 1) - 1) // s + 1
    ref = np.zeros((2, l_out))
    for o in range(2):
        for t in range(l_out):
            acc = float(b[o])
            for i in range(3):
                for j in range(k):
                    n = t * s + j * d - p
                    if 0 <= n < 23:
                        acc += float(w[o, i, j]) * float(x[i, n])
            ref[o, t] = acc
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    tref = F.conv1d(torch.from_numpy(x).double()[None], torch.from_numpy(w).double(), torch.from_numpy(b).double(),
                    stride=s, padding=p, dilation=d)[0].numpy()
    np.testing.assert_allclose(got, tref, rtol=1e-5, atol=1e-5)


def test_snake_closed_forms():
    alpha = np.array([1.0, 2.0, 0.5], dtype=np.float32)
    x = np.array([[math.pi / 2], [math.pi / 4], [math.pi]], dtype=np.float32)   # sin(alpha x) = 1
    np.testing.assert_allclose(O.snake(x, alpha)[:, 0], x[:, 0] + 1.0 / alpha, rtol=1e-6)
    z = np.array([[math.pi], [math.pi / 2], [2 * math.pi]], dtype=np.float32)   # sin(alpha x) = 0
    np.testing.assert_allclose(O.snake(z, alpha)[:, 0], z[:, 0], atol=1e-6)
    np.testing.assert_array_equal(O.snake(np.zeros((3, 4), np.float32), alpha), np.zeros((3, 4), np.float32))


def _torch_encode(params, wave, cfg):
    """The encoder's steps composed from torch CPU float64 ops (conv1d with
    stride / dilation / padding, torch's weight norm, Snake written out)."""
    p = {k: torch.from_numpy(np.asarray(v)).double() for k, v in params.items()}

    def wn(prefix):
        return torch._weight_norm(p[prefix + ".weight_v"], p[prefix + ".weight_g"], 0)

    def snake(x, a):
        a = a.reshape(1, -1, 1)
        return x + torch.sin(a * x) ** 2 / (a + 1e-9)

    x = torch.from_numpy(wave).double()
    hop = int(np.prod(cfg["encoder_rates"]))
    pad = -(-x.shape[-1] // hop) * hop - x.shape[-1]
    x = F.pad(x, (0, pad))
    x = F.conv1d(x, wn("encoder.block.0"), p["encoder.block.0.bias"], padding=3)
    for i, s in enumerate(cfg["encoder_rates"], start=1):
        for u, d in enumerate((1, 3, 9)):
            q = f"encoder.block.{i}.block.{u}"
            r = snake(x, p[q + ".block.0.alpha"])
            r = F.conv1d(r, wn(q + ".block.1"), p[q + ".block.1.bias"], padding=3 * d, dilation=d)
            r = snake(r, p[q + ".block.2.alpha"])
            r = F.conv1d(r, wn(q + ".block.3"), p[q + ".block.3.bias"])
            x = x + r
        x = snake(x, p[f"encoder.block.{i}.block.3.alpha"])
        x = F.conv1d(x, wn(f"encoder.block.{i}.block.4"), p[f"encoder.block.{i}.block.4.bias"], stride=s,
                     padding=math.ceil(s / 2))
    n = len(cfg["encoder_rates"])
    x = snake(x, p[f"encoder.block.{n + 1}.alpha"])
    return F.conv1d(x, wn(f"encoder.block.{n + 2}"), p[f"encoder.block.{n + 2}.bias"], padding=1).numpy()


def test_encode_hidden_matches_torch_composition():
    cfg = dict(O.DEFAULT_CONFIG, **ENC_SMALL)
    params = synth.make_encoder_params(ENC_SMALL, seed=3)
    wave = synth.make_waveform(2, 2 * 800 + 37, seed=3)
    got = O.encode_hidden(params, wave, ENC_SMALL)
    ref = _torch_encode(params, wave, cfg)
    assert got.shape == (2, 16, 3)
    # the oracle rounds every layer's output to fp32 (about 40 of them)
    assert rel_l2(got, ref) < 3e-5


def test_encode_hidden_length_law_and_right_pad():
    params = synth.make_encoder_params(ENC_SMALL, seed=1)
    wave = synth.make_waveform(1, 1601, seed=1)
    h = O.encode_hidden(params, wave, ENC_SMALL)
    assert h.shape == (1, 16, 3)
    padded = np.concatenate([wave, np.zeros((1, 1, 799), np.float32)], axis=2)
    np.testing.assert_array_equal(O.encode_hidden(params, padded, ENC_SMALL), h)
    assert O.encode_hidden(params, wave[:, :, :1600], ENC_SMALL).shape == (1, 16, 2)


def test_encode_hidden_depends_on_a_finite_window():
    # Latent 0 reaches at most ~8.7 k samples past its own 800: perturbing
    # the last 2400 of 16 latents' samples leaves it unchanged, latent 15 not.
    params = synth.make_encoder_params(ENC_SMALL, seed=2)
    wave = synth.make_waveform(1, 16 * 800, seed=2)
    h = O.encode_hidden(params, wave, ENC_SMALL)
    w2 = wave.copy()
    w2[:, :, -2400:] += 0.25
    h2 = O.encode_hidden(params, w2, ENC_SMALL)
    np.testing.assert_array_equal(h2[:, :, 0], h[:, :, 0])
    assert np.max(np.abs(h2[:, :, 15] - h[:, :, 15])) > 1e-3


def test_encode_hidden_batch_items_independent():
    params = synth.make_encoder_params(ENC_SMALL, seed=4)
    wave = synth.make_waveform(3, 1600, seed=4)
    h = O.encode_hidden(params, wave, ENC_SMALL)
    for i in range(3):
        np.testing.assert_array_equal(h[i], O.encode_hidden_item(params, wave[i, 0], ENC_SMALL))


def test_encoder_window_interior_equals_full_encode():
    # a window widened by encoder_margin_frames per side reproduces the full
    # encode on its interior (what the GPU test's sampled windows rely on)
    from tests.conftest import encoder_margin_frames
    rates = O.DEFAULT_CONFIG["encoder_rates"]
    m = encoder_margin_frames(rates)
    assert m == 14
    params = synth.make_encoder_params(ENC_SMALL, seed=5)
    n = 2 * m + 3
    wave = synth.make_waveform(1, n * 800 - 321, seed=5)
    full = O.encode_hidden(params, wave, ENC_SMALL)
    f0, f1 = m, m + 2
    win = O.encode_hidden(params, wave[:, :, (f0 - m) * 800:(f1 + m) * 800], ENC_SMALL)
    np.testing.assert_array_equal(win[:, :, m:m + 2], full[:, :, f0:f1])
    # the right edge: the window ends at the ragged end of the waveform
    win = O.encode_hidden(params, wave[:, :, (n - 1 - m) * 800:], ENC_SMALL)
    np.testing.assert_array_equal(win[:, :, m:], full[:, :, n - 1:])


# ---------------------------------------------------------------------------
# Attention projection pre_block and the posterior mean (FastVideo
# "minimax_h3_audio_vae", module overview, Encoder bullet; diffusers
# "AutoencoderKLMiniMaxH3Audio": is_causal=True, mean_proj)
# ---------------------------------------------------------------------------

PB_SMALL = {"latent_dim": 16, "latent_channels": 4, "num_attention_heads": 2, "mlp_width": 6}


def pre_block_torch(params, hidden, heads, c):
    """The readings written with torch's own routines in float64: F.linear,
    scaled_dot_product_attention with is_causal=True (the mask the diffusers
    page names), a mean over heads, avg_pool1d, F.gelu (exact), conv1d."""
    P = {k: torch.tensor(np.asarray(v, np.float64)) for k, v in params.items()}
    x = torch.tensor(np.asarray(hidden, np.float64)).T  # (N, D)
    n, d = x.shape
    hd = d // heads
    bias = torch.cat([P["pre_block.attn.q_bias"], torch.zeros(d, dtype=F64), P["pre_block.attn.v_bias"]])
    q, k, v = F.linear(x, P["pre_block.attn.qkv.weight"], bias).split(d, dim=1)
    q, k, v = (t.reshape(n, heads, hd).transpose(0, 1) for t in (q, k, v))  # (H, N, hd)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True).mean(dim=0)  # (N, hd)
    a = F.avg_pool1d(o.unsqueeze(1), kernel_size=hd // c).squeeze(1)       # (N, C)
    y = F.linear(a, P["pre_block.attn.proj.weight"], P["pre_block.attn.proj.bias"])
    val, gate = F.linear(y, P["pre_block.mlp.fc1.weight"], P["pre_block.mlp.fc1.bias"]).chunk(2, dim=1)
    m = val * F.gelu(gate, approximate="none")
    y2 = F.linear(m, P["pre_block.mlp.fc2.weight"], P["pre_block.mlp.fc2.bias"])
    return F.conv1d(y2.T.unsqueeze(0), P["mean_proj.weight"], P["mean_proj.bias"])[0].numpy()


@pytest.mark.parametrize("cfg,n", [(PB_SMALL, 13), ({"latent_dim": 64, "latent_channels": 4,
                                                     "num_attention_heads": 8, "mlp_width": 16}, 40)])
def test_pre_block_and_mean_proj_match_torch_composition(cfg, n):
    p = synth.make_pre_block_params(cfg, seed=1)
    hidden = synth.make_signal((cfg["latent_dim"], n), seed=2, scale=100.0)
    proj = O.pre_block_item(p, hidden, cfg)
    got = O.conv1d(proj, p["mean_proj.weight"], p["mean_proj.bias"])
    ref = pre_block_torch(p, hidden, cfg["num_attention_heads"], cfg["latent_channels"])
    assert got.shape == (cfg["latent_channels"], n)
    assert rel_l2(got, ref) < 2e-6  # the oracle rounds six intermediate results to float32


def test_first_token_attends_only_to_itself_and_uniform_scores_give_running_means():
    rng = np.random.default_rng(0)
    n, d, heads = 9, 12, 3
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    o = O.causal_attention_heads_mean(q, k, v, heads)
    hd = d // heads
    # token 0 sees only itself: the mean over heads of its own v
    np.testing.assert_allclose(o[0], v[0].reshape(heads, hd).mean(axis=0), rtol=1e-6)
    # q = 0: every allowed score is 0, the softmax is uniform over u <= t,
    # so each head's output is the running mean of v
    o0 = O.causal_attention_heads_mean(np.zeros_like(q), k, v, heads)
    run = np.cumsum(v.astype(np.float64), axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o0, run.reshape(n, heads, hd).mean(axis=1), rtol=1e-6, atol=1e-7)


def test_identical_heads_average_to_one_head():
    rng = np.random.default_rng(1)
    n, hd, heads = 7, 4, 3
    q1, k1, v1 = (rng.standard_normal((n, hd)).astype(np.float32) for _ in range(3))
    one = O.causal_attention_heads_mean(q1, k1, v1, 1)
    many = O.causal_attention_heads_mean(np.tile(q1, heads), np.tile(k1, heads), np.tile(v1, heads), heads)
    np.testing.assert_allclose(many, one, rtol=1e-6)


def test_attention_is_causal():
    # changing the hidden state at frame t changes no output before t
    p = synth.make_pre_block_params(PB_SMALL, seed=3)
    h = synth.make_signal((16, 11), seed=4, scale=100.0)
    a = O.pre_block_item(p, h, PB_SMALL)
    h2 = h.copy()
    h2[:, 6] += 50.0
    b = O.pre_block_item(p, h2, PB_SMALL)
    np.testing.assert_array_equal(a[:, :6], b[:, :6])
    assert np.abs(a[:, 6:] - b[:, 6:]).max() > 1e-3


def test_k_bias_is_forced_to_zero_and_fused_bias_form():
    p = synth.make_pre_block_params(PB_SMALL, seed=5)
    h = synth.make_signal((16, 8), seed=6, scale=100.0)
    ref = O.pre_block_item(p, h, PB_SMALL)
    fused = {k: v for k, v in p.items() if k not in ("pre_block.attn.q_bias", "pre_block.attn.v_bias")}
    kb = np.full(16, 3.0, np.float32)  # a stored k bias is ignored
    fused["pre_block.attn.qkv.bias"] = np.concatenate([p["pre_block.attn.q_bias"], kb, p["pre_block.attn.v_bias"]])
    np.testing.assert_array_equal(O.pre_block_item(fused, h, PB_SMALL), ref)


def test_gelu_closed_forms_and_geglu_half_order():
    # GELU(x) = x Phi(x): Phi(1) = 0.841344746068543, Phi(2) = 0.977249868051821
    np.testing.assert_allclose(O.gelu([0.0, 1.0, -1.0, 2.0]),
                               [0.0, 0.841344746068543, -0.158655253931457, 1.954499736103642], rtol=1e-13)
    # fc1 rows: the value half reads 1, the gate half reads stream 0; a block
    # whose attention output is constant makes the gate known exactly
    cfg = dict(PB_SMALL, mlp_width=1)
    p = synth.make_pre_block_params(cfg, seed=7)
    p["pre_block.attn.qkv.weight"][:] = 0.0
    p["pre_block.attn.v_bias"][:] = 2.0       # every v is 2 -> every pooled stream is 2
    p["pre_block.attn.proj.weight"][:] = np.eye(4, dtype=np.float32)
    p["pre_block.attn.proj.bias"][:] = 0.0
    p["pre_block.mlp.fc1.weight"][:] = [[0, 0, 0, 0], [0.5, 0, 0, 0]]  # value 0 + 1 (bias), gate 1
    p["pre_block.mlp.fc1.bias"][:] = [1.0, 0.0]
    p["pre_block.mlp.fc2.weight"][:] = 1.0
    p["pre_block.mlp.fc2.bias"][:] = 0.0
    out = O.pre_block_item(p, np.zeros((16, 3), np.float32), cfg)
    np.testing.assert_allclose(out, 0.841344746068543, rtol=1e-6)  # value 1 times GELU(gate 1)
    p["pre_block.mlp.fc1.bias"][:] = [3.0, 0.0]  # value 3, gate 1: 3 GELU(1) = 2.524; swapped halves: GELU(3) = 2.996
    out = O.pre_block_item(p, np.zeros((16, 3), np.float32), cfg)
    np.testing.assert_allclose(out, 3 * 0.841344746068543, rtol=1e-6)


def test_encode_mean_of_items_is_independent_and_composes():
    cfg = dict(PB_SMALL, encoder_dim=4)
    p = dict(synth.make_encoder_params(cfg, seed=8), **synth.make_pre_block_params(cfg, seed=8))
    w = synth.make_waveform(2, 3 * 800 + 5, seed=8)
    m = O.encode(p, w, cfg)
    assert m.shape == (2, 4, 4)
    np.testing.assert_array_equal(m[1], O.encode(p, w[1:2], cfg)[0])
    h = O.encode_hidden(p, w[:1], cfg)[0]
    np.testing.assert_array_equal(m[0], O.conv1d(O.pre_block_item(p, h, cfg), p["mean_proj.weight"],
                                                 p["mean_proj.bias"]))
