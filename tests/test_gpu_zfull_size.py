"""Full-size workloads against the oracle, every output element.

The persistent conv kernel hands its copy pipeline from one output tile to
the next inside a workgroup, which only happens once tiles outnumber
workgroups: these tests compare every unclamped output of the throughput
workloads with the CPU oracle, so that every tile boundary at full size is
checked. The oracle runs in background workers started at collection
(tests/full_oracle.py); the tests sit late in the run so that its minutes
of CPU work overlap the other GPU tests.

Tolerances as everywhere for the fp32 path: relative L2 <= 1e-4 and
max |diff| <= 1e-3 (the encoder's hidden state, a few hundred in magnitude
under random weights, takes 1e-3 * max(1, max|ref| / 10))."""

import numpy as np
import pytest

from neural_audio_vae_amd import synth
from tests import full_oracle as FO

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REL_TOL, ABS_TOL = 1e-4, 1e-3


def check(what, got, ref, abs_tol=ABS_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rl = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    ma = float(np.max(np.abs(got - ref)))
    sat = float(np.mean(np.abs(ref) >= 1.0))
    print(f"[parity] {what}: n={ref.size} (every element) rel_l2={rl:.3e} max_abs={ma:.3e} "
          f"max|ref|={np.max(np.abs(ref)):.3g} |ref|>=1: {sat:.2%}", flush=True)
    assert rl <= REL_TOL and ma <= abs_tol, f"{what}: rel_l2={rl:.3e} max_abs={ma:.3e}"


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def decoder(dev):
    from neural_audio_vae_amd import Decoder
    d = Decoder(synth.make_params())
    yield d
    d.close()


@pytest.fixture(scope="module")
def c4_out(decoder, dev):
    x = synth.make_signal(FO.C4, seed=0)
    print(f"[case] c4 stage-1 AMP set {FO.C4}", flush=True)
    y = decoder.amp_stage(1, torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.fixture(scope="module")
def c3_out(decoder, dev):
    z = synth.make_latents(*FO.C3)
    print(f"[case] c3 decode B={FO.C3[0]} N={FO.C3[1]} unclamped", flush=True)
    y = decoder.decode(torch.from_numpy(z).to(dev), flags=0x4)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.timeout(900)
@pytest.mark.full_oracle("c4/0", "c4/1")
@pytest.mark.parametrize("item", range(FO.C4[0]))
def test_c4_every_output(c4_out, full_oracle, item):
    check(f"c4 item {item}", c4_out[item], full_oracle.result(f"c4/{item}"))


@pytest.mark.timeout(900)
@pytest.mark.full_oracle("c3/0", "c3/1")
@pytest.mark.parametrize("item", range(FO.C3[0]))
def test_c3_every_output(c3_out, full_oracle, item):
    ref = full_oracle.result(f"c3/{item}")
    check(f"c3 item {item} unclamped", c3_out[item], ref)
    check(f"c3 item {item} clamped", np.clip(c3_out[item], -1, 1), np.clip(ref, -1, 1))


@pytest.fixture(scope="module")
def e3_params():
    return dict(synth.make_encoder_params(seed=0), **synth.make_pre_block_params(seed=0))


@pytest.fixture(scope="module")
def e3_out(dev, e3_params):
    """(hidden, posterior mean) of the e3 workload on the GPU."""
    from neural_audio_vae_amd import Encoder
    batch, samples, seed = FO.E3
    enc = Encoder(e3_params)
    print(f"[case] e3 encode B={batch} S={samples}", flush=True)
    wave = torch.from_numpy(synth.make_waveform(batch, samples, seed=seed)).to(dev)
    h = enc.encode_hidden(wave)
    mu = enc.encode_mean(wave)
    torch.cuda.synchronize()
    out = h.cpu().numpy(), mu.cpu().numpy()
    enc.close()
    return out


@pytest.mark.timeout(900)
@pytest.mark.full_oracle(*[f"e3/0/{k}" for k in range(len(FO.E3_WINDOWS))])
def test_e3_item0_every_frame(e3_out, e3_params, full_oracle):
    # item 0's 1200 frames from four oracle windows whose interiors tile it;
    # then the attention projection (causal over all 1200 frames) and
    # mean_proj of the oracle on that hidden state
    import oracle as O
    hidden, mean = e3_out
    parts = [full_oracle.result(f"e3/0/{k}") for k in range(len(FO.E3_WINDOWS))]
    ref = np.concatenate(parts, axis=1)
    assert ref.shape == hidden[0].shape
    check("e3 item 0 hidden", hidden[0], ref, abs_tol=ABS_TOL * max(1.0, float(np.max(np.abs(ref))) / 10.0))
    mref = O.conv1d(O.pre_block_item(e3_params, ref), e3_params["mean_proj.weight"], e3_params["mean_proj.bias"])
    check("e3 item 0 posterior mean", mean[0], mref)
