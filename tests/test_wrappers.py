"""CPU checks of the torch wrappers' argument checks: the C ABI takes raw
device pointers without sizes, so every tensor is checked before a call.
The checks read only tensor metadata; fake CUDA tensors stand in here."""

import pytest

torch = pytest.importorskip("torch")

from neural_audio_vae_amd import decoder as D  # noqa: E402


class FakeCuda:
    """Metadata of a CUDA tensor (no device memory)."""

    def __init__(self, shape, dtype=torch.float32, index=0, contiguous=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.is_cuda = True
        self.device = torch.device("cuda", index)
        self._contiguous = contiguous

    def is_contiguous(self):
        return self._contiguous


def test_check_tensor_accepts_the_expected_tensor():
    D._check_tensor(FakeCuda((2, 32, 5)), "latents", 0, ndim=3)
    D._check_tensor(FakeCuda((2, 1, 4000)), "out", 0, shape=(2, 1, 4000))


@pytest.mark.parametrize("bad,why", [
    (torch.zeros((2, 32, 5)), "CUDA"),                          # host tensor
    (FakeCuda((2, 32, 5), dtype=torch.float64), "float32"),     # wrong dtype
    (FakeCuda((2, 32, 5), index=1), "cuda:1"),                  # another device
    (FakeCuda((32, 5)), "dims"),                                # wrong rank
])
def test_check_tensor_rejects_bad_inputs(bad, why):
    with pytest.raises(ValueError, match=why):
        D._check_tensor(bad, "latents", 0, ndim=3)


@pytest.mark.parametrize("shape", [(2, 1, 3999), (1, 1, 4000), (2, 2, 4000), (2, 4000)])
def test_output_of_the_wrong_shape_is_refused(shape):
    with pytest.raises(ValueError, match="shape"):
        D._output(FakeCuda(shape), "out", 0, (2, 1, 4000), None)


def test_non_contiguous_output_is_refused():
    with pytest.raises(ValueError, match="contiguous"):
        D._output(FakeCuda((2, 1, 4000), contiguous=False), "out", 0, (2, 1, 4000), None)


def test_given_output_is_returned_unchanged():
    out = FakeCuda((2, 1, 4000))
    assert D._output(out, "out", 0, (2, 1, 4000), None) is out
