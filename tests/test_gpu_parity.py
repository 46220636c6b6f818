"""GPU path vs the CPU oracle, through the C ABI.

Tolerances (fp32 path): relative L2 <= 1e-4 and max |diff| <= 1e-3 on both
the clamped waveform and the unclamped signal (MH3A_FLAG_NO_CLAMP); most
samples saturate under random weights, so the unclamped comparison is the
sharp one. bf16 matrix-core operands: relative L2 <= 2e-2.

Full-size workloads are checked on sampled output windows: the oracle
decodes only the latents within the receptive radius of each window, whose
interior equals the full decode (pinned in test_oracle_pins.py)."""

import functools
import math
import sys

import numpy as np
import pytest

import oracle as O
from neural_audio_vae_amd import synth
from tests.conftest import SMALL_CONFIG

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REL_TOL, ABS_TOL, BF16_REL_TOL = 1e-4, 1e-3, 2e-2
# The absolute bound is stated for the five workloads, whose signals stay
# below ~10 in magnitude. The extra configurations (other widths, random
# weight-norm gains, custom filters) produce larger signals; for them the
# absolute bound scales with the signal: 1e-3 * max(1, max|ref| / 10).
REF_SCALE = 10.0


def scaled_abs(ref):
    return ABS_TOL * max(1.0, float(np.max(np.abs(ref))) / REF_SCALE)


NO_CLAMP, BF16, DENORM, INVARIANT = 0x4, 0x2, 0x1, 0x8


def report(what, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rl = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    ma = float(np.max(np.abs(got - ref))) if got.size else 0.0
    sat = float(np.mean(np.abs(ref) >= 1.0)) if ref.size else 0.0
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    print(f"[parity] {what}: n={ref.size} rel_l2={rl:.3e} max_abs={ma:.3e} max|ref|={mx:.3g} |ref|>=1: {sat:.2%}",
          flush=True)
    return rl, ma


def assert_close(what, got, ref, rel=REL_TOL, abs_=ABS_TOL):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rl, ma = report(what, got, ref)
    assert rl <= rel and ma <= abs_, f"{what}: rel_l2={rl:.3e} max_abs={ma:.3e}"


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def default_decoder(default_params, dev):
    from neural_audio_vae_amd import Decoder
    mean, std = synth.make_denorm()
    d = Decoder(default_params, latents_mean=mean, latents_std=std)
    yield d
    d.close()


@pytest.fixture(scope="module")
def small_decoder(small_params, dev):
    from neural_audio_vae_amd import Decoder
    d = Decoder(small_params, SMALL_CONFIG)
    yield d
    d.close()


def gpu(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ---------------------------------------------------------------------------
# Narrow decoder: full decodes, many lengths, both flags
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("batch,frames", [(1, 1), (1, 2), (2, 3), (1, 7), (3, 13)])
def test_small_decoder_full_decode(small_decoder, small_params, dev, batch, frames):
    z = synth.make_latents(batch, frames, seed=frames, channels=4)
    ref = O.decode(small_params, z, SMALL_CONFIG, clamp=False)
    got = host(small_decoder.decode(gpu(z, dev), flags=NO_CLAMP))
    assert_close(f"small B={batch} N={frames} unclamped", got, ref, abs_=scaled_abs(ref))
    got_c = host(small_decoder.decode(gpu(z, dev)))
    assert_close(f"small B={batch} N={frames} clamped", got_c, np.clip(ref, -1, 1))
    assert np.all(np.abs(got_c) <= 1.0)


def test_small_decoder_nan_latent_propagates_like_the_oracle(small_decoder, small_params, dev):
    # A NaN latent (a degenerate input) turns the samples within the
    # decoder's receptive radius into NaN, clamped or not (the clamp keeps
    # NaN, as the pages' torch.clamp / mx.clip do), and the samples outside
    # it decode as usual. Every sample the oracle makes NaN is NaN here too.
    # The transposed convs of rate 5 and kernel 9 run each phase as two taps
    # and phase 2 has one real tap, so its zero-weight slot multiplies a
    # neighbouring input: at the edge of a NaN region 0 * NaN widens the NaN
    # band by a few samples (less than one latent, 800 samples).
    z = synth.make_latents(1, 80, seed=11, channels=4)
    z[0, 2, 5] = np.nan
    ref = O.decode(small_params, z, SMALL_CONFIG, clamp=False)
    bad = np.isnan(ref)
    assert bad.any() and not bad.all()
    idx = np.nonzero(bad[0, 0])[0]
    lo, hi = int(idx.min()), int(idx.max())
    assert idx.size == hi - lo + 1  # one contiguous region
    for flags, r in ((NO_CLAMP, ref), (0, O.decode(small_params, z, SMALL_CONFIG, clamp=True))):
        got = host(small_decoder.decode(gpu(z, dev), flags=flags))
        gbad = np.isnan(got)
        assert gbad[bad].all(), "every oracle NaN is NaN on the GPU"
        extra = np.nonzero(gbad[0, 0] & ~bad[0, 0])[0]
        print(f"[parity] NaN latent flags={flags}: oracle NaN [{lo}, {hi}], GPU-only NaN {extra.size}"
              + (f" in [{extra.min()}, {extra.max()}]" if extra.size else ""), flush=True)
        assert np.all((extra >= lo - 800) & (extra <= hi + 800)) and extra.size < 800
        ok = ~gbad
        assert_close(f"small NaN latent flags={flags} (finite samples)", got[ok], r[ok], abs_=scaled_abs(r[ok]))


def test_fp16_piece_form_out_of_range_gives_nan_and_the_bf16x6_form_matches(small_decoder, small_params, dev):
    # The default matrix form splits every conv input of the wide stages into
    # two fp16 pieces, which holds while the inputs stay below fp16's 65504.
    # Latents scaled by 1e5 drive the layer outputs to ~1e5 (the oracle stays
    # finite): the default form then returns NaN samples, clamped or not,
    # never finite wrong ones, while the six-product bf16 form (fp32's range)
    # matches the oracle.
    from neural_audio_vae_amd import Decoder, _lib
    z = (synth.make_latents(1, 6, seed=12, channels=4) * np.float32(1e5)).astype(np.float32)
    ref, stages = O.decode_item(small_params, z[0], SMALL_CONFIG, clamp=False, return_stages=True)
    ref = ref[None]
    assert np.isfinite(ref).all() and max(float(np.abs(s).max()) for s in stages) > 65504
    for flags in (NO_CLAMP, 0):
        got = host(small_decoder.decode(gpu(z, dev), flags=flags))
        nan = np.isnan(got)
        print(f"[parity] fp16 form, latents x1e5, flags={flags}: NaN samples {int(nan.sum())} of {nan.size}", flush=True)
        assert nan.any() and np.isfinite(got[~nan]).all()
        if (~nan).any():
            r = ref if flags else np.clip(ref, -1, 1)
            assert_close(f"fp16 form x1e5 flags={flags} (finite samples)", got[~nan], r[~nan], abs_=scaled_abs(r[~nan]))
    d6 = Decoder(small_params, dict(SMALL_CONFIG, matrix_form=_lib.MH3A_MATRIX_SPLIT))
    got6 = host(d6.decode(gpu(z, dev), flags=NO_CLAMP))
    d6.close()
    assert_close("bf16x6 form, latents x1e5", got6, ref, abs_=scaled_abs(ref))


def test_small_decoder_fold_uses_axis0_of_each_weight(dev):
    # g drawn away from ||v||: the fold changes every weight, per output
    # channel for convs and per input channel for the transposed convs.
    from neural_audio_vae_amd import Decoder
    p = synth.make_params(SMALL_CONFIG, seed=5, g_mode="uniform")
    d = Decoder(p, SMALL_CONFIG)
    z = synth.make_latents(2, 5, seed=5, channels=4)
    ref = O.decode(p, z, SMALL_CONFIG, clamp=False)
    assert_close("small random-g", host(d.decode(gpu(z, dev), flags=NO_CLAMP)), ref, abs_=scaled_abs(ref))
    d.close()


def test_small_decoder_given_filters_and_folded_weights(dev):
    # Filter buffers passed with the parameters replace the designed taps,
    # and an already folded `.weight` replaces weight_v / weight_g.
    from neural_audio_vae_amd import Decoder
    p = dict(synth.make_params(SMALL_CONFIG, seed=6))
    rng = np.random.default_rng(0)
    for name in ("decoder.resblocks.2.activations.1", "decoder.resblocks.19.activations.4", "decoder.activation_post"):
        f = rng.uniform(-0.2, 0.6, size=12).astype(np.float32)
        p[name + ".upsample.filter"] = f
        p[name + ".downsample.lowpass.filter"] = f[::-1].copy()
    pre = "decoder.resblocks.7.convs2.1"
    p[pre + ".weight"] = O.fold_weight_norm(p.pop(pre + ".weight_v"), p.pop(pre + ".weight_g"))
    del p["decoder.conv_post.bias"]
    d = Decoder(p, SMALL_CONFIG)
    z = synth.make_latents(1, 6, seed=6, channels=4)
    ref = O.decode(p, z, SMALL_CONFIG, clamp=False)
    assert_close("small custom filters", host(d.decode(gpu(z, dev), flags=NO_CLAMP)), ref, abs_=scaled_abs(ref))
    d.close()


def test_small_decoder_other_shapes(dev):
    # A different stage layout: two stages, one block, two dilations.
    from neural_audio_vae_amd import Decoder
    cfg = {"latent_channels": 3, "latent_dim": 20, "decoder_dim": 40, "decoder_rates": (4, 3),
           "decoder_kernel_sizes": (8, 7), "resblock_kernel_sizes": (5,), "resblock_dilation_sizes": ((2, 7),),
           "hop_length": 12}
    p = synth.make_params(cfg, seed=8)
    d = Decoder(p, cfg)
    z = synth.make_latents(2, 9, seed=8, channels=3)
    ref = O.decode(p, z, cfg, clamp=False)
    assert_close("custom config", host(d.decode(gpu(z, dev), flags=NO_CLAMP)), ref, abs_=scaled_abs(ref))
    d.close()


# ---------------------------------------------------------------------------
# Default decoder, c1: every layer, then the output
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def c1_oracle_stages():
    p = synth.make_params()
    z = synth.make_latents(1, 4)
    y, stages = O.decode_item(p, z[0], clamp=False, return_stages=True)
    return z, y, stages


def test_c1_every_layer(default_decoder, dev):
    z, _, stages = c1_oracle_stages()
    zt = gpu(z, dev)
    for upto, ref in enumerate(stages):
        got = host(default_decoder.decode_partial(zt, upto))[0]
        assert_close(f"c1 layer {upto}", got, ref)


def test_c1_decode(default_decoder, dev):
    z, y, _ = c1_oracle_stages()
    got = host(default_decoder.decode(gpu(z, dev), flags=NO_CLAMP))
    assert_close("c1 unclamped", got[0], y)
    got_c = host(default_decoder.decode(gpu(z, dev)))
    assert_close("c1 clamped", got_c[0], np.clip(y, -1, 1))


def test_c1_bf16_variant(default_decoder, dev):
    z, y, _ = c1_oracle_stages()
    got = host(default_decoder.decode(gpu(z, dev), flags=NO_CLAMP | BF16))
    assert_close("c1 bf16 unclamped", got[0], y, rel=BF16_REL_TOL, abs_=math.inf)


# ---------------------------------------------------------------------------
# Full-size workloads on sampled windows
# ---------------------------------------------------------------------------

def oracle_windows(params, z, windows, denorm=None):
    """[(item, n0, n1)] -> list of oracle outputs (1, 800 (n1 - n0))."""
    out = []
    for item, n0, n1 in windows:
        kw = {}
        if denorm is not None:
            kw = dict(denormalize=True, latents_mean=denorm[0], latents_std=denorm[1])
        out.append(O.decode_window(params, z[item:item + 1], n0, n1, clamp=False, **kw)[0, 0])
    return out


def check_windows(tag, got, refs, windows, rel=REL_TOL, abs_=ABS_TOL):
    for (item, n0, n1), ref in zip(windows, refs):
        g = got[item, 0, 800 * n0:800 * n1]
        assert_close(f"{tag} item {item} latents [{n0},{n1}) unclamped", g, ref, rel, abs_)


@pytest.mark.parametrize("cfg", ["c2", "c3", "c5"])
def test_full_size_sampled_windows(default_decoder, default_params, dev, cfg):
    if cfg == "c2":
        batch, frames, flags = 2, 200, DENORM
        denorm = synth.make_denorm()
        windows = [(0, 0, 3), (1, 100, 103), (1, 197, 200)]
    elif cfg == "c3":
        batch, frames, flags, denorm = 2, 1200, 0, None
        windows = [(0, 0, 2), (0, 600, 603), (1, 1198, 1200)]
    else:
        batch, frames, flags, denorm = 16, 401, 0, None
        windows = [(0, 0, 2), (7, 200, 203), (15, 399, 401)]
    z = synth.make_latents(batch, frames)
    print(f"[case] {cfg} B={batch} N={frames} flags={flags}", flush=True)
    out = default_decoder.decode(gpu(z, dev), flags=flags | NO_CLAMP)
    got = host(out)
    assert got.shape == (batch, 1, 800 * frames)
    assert np.all(np.isfinite(got))
    refs = oracle_windows(default_params, z, windows, denorm)
    check_windows(cfg, got, refs, windows)
    clamped = host(default_decoder.decode(gpu(z, dev), flags=flags))
    np.testing.assert_array_equal(clamped, np.clip(got, -1, 1))


def test_c3_bf16_variant_sampled(default_decoder, default_params, dev):
    z = synth.make_latents(2, 1200)
    windows = [(0, 600, 602), (1, 0, 2)]
    got = host(default_decoder.decode(gpu(z, dev), flags=NO_CLAMP | BF16))
    refs = oracle_windows(default_params, z, windows)
    check_windows("c3 bf16", got, refs, windows, rel=BF16_REL_TOL, abs_=math.inf)


def test_c4_amp_stage_microbench(default_decoder, default_params, dev):
    # Stage-1 AMP set alone on (2, 256, 30000) ~ N(0, 1); checked on
    # windows whose margin (120 samples) exceeds the set's radius (90).
    x = synth.make_signal((2, 256, 30000), seed=0)
    got = host(default_decoder.amp_stage(1, gpu(x, dev)))
    assert got.shape == x.shape
    margin = 120
    for item, a, b in [(0, 0, 64), (1, 15000, 15064), (1, 29936, 30000), (0, 29990, 30000)]:
        lo, hi = max(0, a - margin), min(30000, b + margin)
        ref = O.stage_amp(x[item][:, lo:hi], default_params, 1)[:, a - lo:b - lo]
        assert_close(f"c4 item {item} [{a},{b})", got[item][:, a:b], ref)


def test_stage0_packed_activation_path(default_decoder, default_params, dev):
    # Stage 0 (512 channels) on (1, 512, 3000): large enough that each conv
    # takes its activated input from the standalone pass (packed, zero
    # padded), including the tiles that overhang both ends.
    x = synth.make_signal((1, 512, 3000), seed=5)
    got = host(default_decoder.amp_stage(0, gpu(x, dev)))
    margin = 120
    for a, b in [(0, 48), (1500, 1548), (2952, 3000)]:
        lo, hi = max(0, a - margin), min(3000, b + margin)
        ref = O.stage_amp(x[0][:, lo:hi], default_params, 0)[:, a - lo:b - lo]
        assert_close(f"stage 0 packed [{a},{b})", got[0][:, a:b], ref)


@pytest.mark.parametrize("stage,channels", [(4, 32), (5, 16), (6, 8)])
def test_narrow_stage_windows(default_decoder, default_params, dev, stage, channels):
    # Stages of <= 16 channels run on 16-row tiles (v_mfma_f32_16x16x4f32),
    # 32 channels on 32-row tiles; (2, C, 3000) with windows at both ends.
    x = synth.make_signal((2, channels, 3000), seed=10 + stage)
    got = host(default_decoder.amp_stage(stage, gpu(x, dev)))
    margin = 120
    for item, a, b in [(0, 0, 64), (1, 1400, 1464), (1, 2936, 3000)]:
        lo, hi = max(0, a - margin), min(3000, b + margin)
        ref = O.stage_amp(x[item][:, lo:hi], default_params, stage)[:, a - lo:b - lo]
        assert_close(f"stage {stage} item {item} [{a},{b})", got[item][:, a:b], ref)


def test_amp_stage_rejects_bad_arguments(default_decoder, dev):
    from neural_audio_vae_amd import MH3AError
    x = torch.zeros((1, 256, 50), device=dev)
    with pytest.raises(ValueError):
        default_decoder.amp_stage(7, x)  # no stage 7
    with pytest.raises(MH3AError):
        default_decoder.amp_stage(1, x, flags=0x1)
    # the wrappers check what the C ABI cannot: channels and output shapes
    with pytest.raises(ValueError, match="channels"):
        default_decoder.amp_stage(1, torch.zeros((1, 128, 50), device=dev))
    with pytest.raises(ValueError, match="shape"):
        default_decoder.amp_stage(1, x, out=torch.empty((1, 256, 49), device=dev))
    z = torch.zeros((1, 32, 4), device=dev)
    with pytest.raises(ValueError, match="shape"):
        default_decoder.decode(z, out=torch.empty((1, 1, 3199), device=dev))
    with pytest.raises(ValueError, match="float32"):
        default_decoder.decode(z, out=torch.empty((1, 1, 3200), device=dev, dtype=torch.float64))
    with pytest.raises(ValueError, match="channels"):
        default_decoder.decode(torch.zeros((1, 16, 4), device=dev))


# ---------------------------------------------------------------------------
# Batch semantics and determinism
# ---------------------------------------------------------------------------

def test_batch_invariant_flag_items_decode_bitwise_alike(default_decoder, default_params, dev):
    # With MH3A_FLAG_BATCH_INVARIANT every launch is planned from one item's
    # shape, so an item's output does not depend on the batch it rides in.
    z = synth.make_latents(3, 37, seed=2)
    both = host(default_decoder.decode(gpu(z, dev), flags=NO_CLAMP | INVARIANT))
    for i in range(3):
        one = host(default_decoder.decode(gpu(z[i:i + 1], dev), flags=NO_CLAMP | INVARIANT))
        np.testing.assert_array_equal(both[i], one[0])
    windows = [(1, 17, 20)]
    check_windows("batch-invariant B=3 N=37", both, oracle_windows(default_params, z, windows), windows)


def test_default_plans_agree_across_batch_sizes(default_decoder, dev):
    # Default plans split the contraction by the batch's size; items then
    # agree across batch sizes to rounding, not bitwise.
    z = synth.make_latents(3, 37, seed=2)
    both = host(default_decoder.decode(gpu(z, dev), flags=NO_CLAMP))
    for i in range(3):
        one = host(default_decoder.decode(gpu(z[i:i + 1], dev), flags=NO_CLAMP))
        assert_close(f"B=3 item {i} vs B=1", both[i], one[0])


@pytest.mark.parametrize("flags", [0, INVARIANT])
def test_amp_stage_short_signal_split_contraction(default_decoder, default_params, dev, flags):
    # Stage 0 on a short signal: few output tiles, so the contraction over
    # 512 channels is split into ranges and summed by the reduce pass.
    x = synth.make_signal((1, 512, 150), seed=4)
    got = host(default_decoder.amp_stage(0, gpu(x, dev), flags=flags))
    ref = O.stage_amp(x[0], default_params, 0)
    assert_close(f"stage 0 (1, 512, 150) flags {flags}", got[0], ref)


def test_decode_is_deterministic(default_decoder, dev):
    z = gpu(synth.make_latents(2, 33, seed=3), dev)
    a = host(default_decoder.decode(z, flags=NO_CLAMP))
    b = host(default_decoder.decode(z, flags=NO_CLAMP))
    np.testing.assert_array_equal(a, b)


def test_decode_argument_errors(default_decoder, dev):
    from neural_audio_vae_amd import _lib
    z = gpu(synth.make_latents(1, 4), dev)
    out = torch.empty((1, 1, 3200), device=dev)
    need = default_decoder.workspace_size(1, 4)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    h = default_decoder._h
    st = torch.cuda.current_stream().cuda_stream
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode(h, z.data_ptr(), 1, 4, out.data_ptr(), ws.data_ptr(), need - 1, 0, st)
    assert e.value.code == _lib.MH3A_E_WORKSPACE
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode(h, z.data_ptr(), 1, 4, out.data_ptr(), ws.data_ptr() + 4, need, 0, st)
    assert e.value.code == _lib.MH3A_E_WORKSPACE
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode(h, z.data_ptr(), 0, 4, out.data_ptr(), ws.data_ptr(), need, 0, st)
    assert e.value.code == _lib.MH3A_E_INVALID_ARG
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode(h, z.data_ptr(), 1, 4, out.data_ptr(), ws.data_ptr(), need, 0x80, st)
    assert e.value.code == _lib.MH3A_E_INVALID_ARG
    with pytest.raises(_lib.MH3AError):
        default_decoder.decode_partial(z, 16)
    # the good call still works afterwards
    _lib.mh3a_decode(h, z.data_ptr(), 1, 4, out.data_ptr(), ws.data_ptr(), need, 0, st)
    torch.cuda.synchronize()
    print("[case] argument errors ok", file=sys.stderr)


# ---------------------------------------------------------------------------
# Time-chunked decode (bounded memory, overlap-and-crop)
# ---------------------------------------------------------------------------

def test_small_decoder_chunked_matches_oracle(small_decoder, small_params, dev):
    # Every chunking of N = 90 latents, including one-latent chunks (each a
    # window cut at both ends), a chunk that does not divide N and chunks
    # at least N long, reproduces the oracle's full decode.
    z = synth.make_latents(2, 90, seed=11, channels=4)
    ref = O.decode(small_params, z, SMALL_CONFIG, clamp=False)
    m = small_decoder.margin()
    assert m >= math.ceil(O.receptive_radius_latents(SMALL_CONFIG)) + 1
    for cf in (1, 7, 25, 89, 90, 200):
        print(f"[case] small chunked N=90 chunk={cf} margin={m}", flush=True)
        got = host(small_decoder.decode_chunked(gpu(z, dev), cf, flags=NO_CLAMP))
        assert_close(f"small chunked chunk={cf}", got, ref, abs_=scaled_abs(ref))


def test_chunked_decode_full_size(default_decoder, default_params, dev):
    # (2, 32, 300) in chunks of 64 (last chunk 44 latents), dequantised
    # latents: against the whole-sequence decode everywhere, and against the
    # oracle on windows that straddle chunk boundaries.
    z = synth.make_latents(2, 300, seed=4)
    denorm = synth.make_denorm()
    flags = DENORM | NO_CLAMP
    print("[case] chunked full-size B=2 N=300 chunk=64", flush=True)
    full = host(default_decoder.decode(gpu(z, dev), flags=flags))
    got = host(default_decoder.decode_chunked(gpu(z, dev), 64, flags=flags))
    assert_close("chunked vs whole decode", got, full)
    windows = [(0, 62, 66), (1, 254, 258), (1, 296, 300)]
    refs = oracle_windows(default_params, z, windows, denorm)
    check_windows("chunked", got, refs, windows)
    # chunks covering the sequence are the whole decode itself
    one = host(default_decoder.decode_chunked(gpu(z, dev), 300, flags=flags))
    np.testing.assert_array_equal(one, full)
    clamped = host(default_decoder.decode_chunked(gpu(z, dev), 64, flags=DENORM))
    assert np.all(np.abs(clamped) <= 1.0)


def test_chunked_workspace_is_bounded(default_decoder, dev):
    from neural_audio_vae_amd import _lib
    h = default_decoder._h
    m = default_decoder.margin()
    a = _lib.mh3a_decode_chunked_workspace_size(h, 2, 1000, 64, 0)
    b = _lib.mh3a_decode_chunked_workspace_size(h, 2, 100000, 64, 0)
    assert a == b
    assert a < _lib.mh3a_decode_workspace_size(h, 2, 1000, 0)
    # a window never exceeds chunk + 2 margin latents
    assert a >= _lib.mh3a_decode_workspace_size(h, 2, 64 + 2 * m, 0)


def test_chunked_decode_argument_errors(default_decoder, dev):
    from neural_audio_vae_amd import _lib
    h = default_decoder._h
    z = gpu(synth.make_latents(1, 100), dev)
    out = torch.empty((1, 1, 80000), device=dev)
    need = _lib.mh3a_decode_chunked_workspace_size(h, 1, 100, 16, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode_chunked(h, z.data_ptr(), 1, 100, 0, out.data_ptr(), ws.data_ptr(), need, 0, st)
    assert e.value.code == _lib.MH3A_E_INVALID_ARG
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode_chunked(h, z.data_ptr(), 1, 100, 16, out.data_ptr(), ws.data_ptr(), need - 1, 0, st)
    assert e.value.code == _lib.MH3A_E_WORKSPACE
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode_chunked(h, z.data_ptr(), 1, 100, 16, out.data_ptr(), ws.data_ptr(), need, 0x80, st)
    assert e.value.code == _lib.MH3A_E_INVALID_ARG
    _lib.mh3a_decode_chunked(h, z.data_ptr(), 1, 100, 16, out.data_ptr(), ws.data_ptr(), need, 0, st)
    torch.cuda.synchronize()
    print("[case] chunked argument errors ok", file=sys.stderr)


# ---------------------------------------------------------------------------
# The other matrix-core forms (matrix_form fixed at create): fp32 matrix
# cores throughout, and bf16 pieces with six products; the default (fp16
# pieces, three products) runs everywhere else in this file.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("form", ["fp32", "bf16x6"])
def test_other_matrix_core_forms(default_params, dev, form):
    # fp32: packed fp32 input at 512 channels, fused activation at 256 on
    # this short signal, fp32 unit kernel, plain-row conv_pre and transposed
    # convs; bf16x6: the split-product convs on three bf16 pieces
    from neural_audio_vae_amd import Decoder, _lib
    mf = {"fp32": _lib.MH3A_MATRIX_FP32, "bf16x6": _lib.MH3A_MATRIX_SPLIT}[form]
    print(f"[case] matrix form {form} (matrix_form = {mf})", flush=True)
    d = Decoder(default_params, {"matrix_form": mf})
    z, y, _ = c1_oracle_stages()
    got = host(d.decode(gpu(z, dev), flags=NO_CLAMP))
    assert_close(f"{form} form c1 decode", got[0], y)
    for stage, c in ((0, 512), (1, 256), (4, 32)):
        x = synth.make_signal((1, c, 3000), seed=stage)
        out = host(d.amp_stage(stage, gpu(x, dev)))
        ref = O.stage_amp(x[0][:, 1380:1684], default_params, stage)[:, 120:184]  # 120 samples of margin
        assert_close(f"{form} form stage {stage} [1500,1564)", out[0][:, 1500:1564], ref)
    if form == "bf16x6":
        z3 = synth.make_latents(2, 1200)
        windows = [(0, 600, 603), (1, 1198, 1200)]
        got = host(d.decode(gpu(z3, dev), flags=NO_CLAMP))
        check_windows("bf16x6 form c3", got, oracle_windows(default_params, z3, windows), windows)
    d.close()


def _graph_replays_match(run_eager, run_into, out_shape, make_inputs, dev):
    """Capture one call on a side stream into a HIP graph and replay it
    three times, with eager work of the same library and synchronizations
    between the replays; every replay must equal the eager result bitwise
    (same plans, same kernels)."""
    x0 = make_inputs(0)
    ref0 = run_eager(x0)
    static_x = x0.clone()
    static_out = torch.empty(out_shape, dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_into(static_x, static_out, s)  # warm-up outside capture: plans, workspace
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_into(static_x, static_out, s)
    torch.cuda.synchronize()
    for rep in range(3):
        xr = make_inputs(rep + 1)
        static_x.copy_(xr)
        g.replay()
        torch.cuda.synchronize()
        ref = run_eager(xr)  # eager work between the replays
        torch.cuda.synchronize()
        np.testing.assert_array_equal(static_out.cpu().numpy(), ref.cpu().numpy())
    np.testing.assert_array_equal(run_eager(x0).cpu().numpy(), ref0.cpu().numpy())


def test_decode_replays_from_a_hip_graph(small_decoder, dev):
    # the decode enqueues only kernels on the caller's stream (no memset,
    # allocation or synchronization), so it can be captured and replayed
    print("[case] decode captured in a HIP graph, 3 replays vs eager", flush=True)

    def inputs(seed):
        return torch.from_numpy(synth.make_latents(2, 5, seed=seed, channels=4)).cuda()

    _graph_replays_match(lambda z: small_decoder.decode(z, flags=NO_CLAMP),
                         lambda z, out, s: small_decoder.decode(z, flags=NO_CLAMP, out=out, stream=s),
                         (2, 1, 4000), inputs, dev)


def test_encode_replays_from_a_hip_graph(dev):
    from neural_audio_vae_amd import Encoder
    cfg = {"encoder_dim": 4, "latent_dim": 16}
    enc = Encoder(synth.make_encoder_params(cfg, seed=5), cfg)
    print("[case] encode captured in a HIP graph, 3 replays vs eager", flush=True)

    def inputs(seed):
        return torch.from_numpy(synth.make_waveform(2, 2000, seed=seed)).cuda()

    _graph_replays_match(lambda w: enc.encode_hidden(w), lambda w, out, s: enc.encode_hidden(w, out=out, stream=s),
                         (2, 16, 3), inputs, dev)
    enc.close()
