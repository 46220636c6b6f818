"""mh3a_decode_noalloc (the decode with its intermediates in the library's
static device scratch, for callers that cannot allocate) against
mh3a_decode with a workspace, through the C ABI: two calls in a row, the
second with a smaller input, each equal to the workspace decode (same
kernels, same plans: bitwise, which is within the fp32 tolerance)."""

import numpy as np
import pytest

from neural_audio_vae_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dec():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from neural_audio_vae_amd import Decoder
    mean, std = synth.make_denorm()
    d = Decoder(synth.make_params(), latents_mean=mean, latents_std=std)
    yield d
    d.close()


def decode_ws(d, z, flags):
    from neural_audio_vae_amd import _lib
    b, _, n = z.shape
    out = torch.empty((b, 1, 800 * n), device="cuda")
    need = _lib.mh3a_decode_workspace_size(d._h, b, n, flags)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    _lib.mh3a_decode(d._h, z.data_ptr(), b, n, out.data_ptr(), ws.data_ptr(), need, flags, st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), need


def decode_static(d, z, flags):
    from neural_audio_vae_amd import _lib
    b, _, n = z.shape
    out = torch.full((b, 1, 800 * n), float("nan"), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    _lib.mh3a_decode_noalloc(d._h, z.data_ptr(), b, n, out.data_ptr(), flags, st)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_decode_equals_workspace_decode_twice(dec):
    from neural_audio_vae_amd import _lib
    # the second call smaller than the first: the scratch keeps the first
    # call's contents, which the second must not depend on
    for (b, n, flags) in ((2, 60, 0x1 | 0x4), (1, 7, 0x4)):
        print(f"[case] noalloc decode B={b} N={n} flags={flags:#x}", flush=True)
        z = torch.from_numpy(synth.make_latents(b, n, seed=n)).cuda()
        ref, need = decode_ws(dec, z, flags)
        assert need <= _lib.MH3A_NOALLOC_SCRATCH_BYTES
        got = decode_static(dec, z, flags)
        assert np.all(np.isfinite(got))
        rl = float(np.linalg.norm(got.astype(np.float64) - ref) / np.linalg.norm(ref.astype(np.float64)))
        print(f"[parity] noalloc vs workspace decode B={b} N={n}: rel_l2={rl:.3e} "
              f"max_abs={np.max(np.abs(got - ref)):.3e} (workspace {need} bytes)", flush=True)
        np.testing.assert_array_equal(got, ref)


def test_noalloc_refuses_decodes_beyond_the_scratch(dec):
    from neural_audio_vae_amd import _lib
    z = torch.zeros((2, 32, 1200), device="cuda")
    out = torch.empty((2, 1, 960000), device="cuda")
    assert _lib.mh3a_decode_workspace_size(dec._h, 2, 1200, 0) > _lib.MH3A_NOALLOC_SCRATCH_BYTES
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode_noalloc(dec._h, z.data_ptr(), 2, 1200, out.data_ptr(), 0, None)
    assert e.value.code == _lib.MH3A_E_WORKSPACE
    with pytest.raises(_lib.MH3AError) as e:
        _lib.mh3a_decode_noalloc(dec._h, z.data_ptr(), 0, 4, out.data_ptr(), 0, None)
    assert e.value.code == _lib.MH3A_E_INVALID_ARG
    torch.cuda.synchronize()
