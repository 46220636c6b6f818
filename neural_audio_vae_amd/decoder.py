"""Decoder: torch-tensor convenience over the mh3a C ABI.

torch supplies device memory and the stream; every step of the decode runs
in the library's HIP kernels.
"""

from __future__ import annotations

import numpy as np

from . import _lib
from ._lib import (MH3A_FLAG_BATCH_INVARIANT, MH3A_FLAG_BF16_MFMA, MH3A_FLAG_DENORMALIZE,  # noqa: F401
                   MH3A_FLAG_NO_CLAMP, MH3AError)  # noqa: F401


def _torch():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("mh3a decodes on a ROCm GPU; torch.cuda is not available")
    return torch


class Decoder:
    """A decoder built once from host parameters (weight norm folded and
    filters designed at construction).

    The decode only enqueues kernels on the given stream (no allocation,
    memset or synchronization inside), so a call can be captured into a HIP
    graph (torch.cuda.graph) once a first call of the same shape has sized
    the workspace; workspaces are kept until close()."""

    def __init__(self, params, config=None, latents_mean=None, latents_std=None, device=0):
        self.config = dict(config or {})
        self.device = int(device)
        cfg = _lib.make_config(self.config)
        self.latent_channels = cfg.latent_channels
        self.hop = cfg.hop_length
        self.num_ups = cfg.num_ups
        self._h = _lib.mh3a_decoder_create(cfg, params, latents_mean, latents_std, self.device)
        self._ws = None
        self._old_ws = []

    def close(self):
        if getattr(self, "_h", None):
            _lib.mh3a_destroy(self._h)
            self._h = None
        self._ws, self._old_ws = None, []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _workspace(self, nbytes):
        torch = _torch()
        if self._ws is None or self._ws.numel() < nbytes:
            # a captured HIP graph may still use the previous buffer: keep it
            # until close()
            if self._ws is not None:
                self._old_ws.append(self._ws)
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=f"cuda:{self.device}")
        return self._ws

    @staticmethod
    def _check_input(t, ndim, name):
        torch = _torch()
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.float32 and t.dim() == ndim):
            raise ValueError(f"{name} must be a float32 CUDA tensor with {ndim} dims")
        return t.contiguous()

    def workspace_size(self, batch, frames, flags=0):
        return _lib.mh3a_decode_workspace_size(self._h, batch, frames, flags)

    def decode(self, latents, flags=0, out=None, stream=None):
        torch = _torch()
        z = self._check_input(latents, 3, "latents")
        b, c, n = z.shape
        if c != self.latent_channels:
            raise ValueError(f"latents must have {self.latent_channels} channels")
        if out is None:
            out = torch.empty((b, 1, self.hop * n), dtype=torch.float32, device=z.device)
        nbytes = self.workspace_size(b, n, flags)
        ws = self._workspace(nbytes)
        st = (stream or torch.cuda.current_stream(z.device)).cuda_stream
        _lib.mh3a_decode(self._h, z.data_ptr(), b, n, out.data_ptr(), ws.data_ptr(), ws.numel(), flags, st)
        return out

    def timing(self, enable):
        _lib.mh3a_timing_enable(self._h, enable)

    def timing_read(self):
        return _lib.mh3a_timing_read(self._h)

    def layer_shape(self, frames, upto):
        return _lib.mh3a_decode_layer_shape(self._h, frames, upto)

    def decode_partial(self, latents, upto, flags=0):
        torch = _torch()
        z = self._check_input(latents, 3, "latents")
        b, c, n = z.shape
        ch, length = self.layer_shape(n, upto)
        out = torch.empty((b, ch, length), dtype=torch.float32, device=z.device)
        ws = self._workspace(self.workspace_size(b, n, flags))
        st = torch.cuda.current_stream(z.device).cuda_stream
        _lib.mh3a_decode_partial(self._h, z.data_ptr(), b, n, upto, out.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                                 st)
        return out

    def margin(self):
        """Latents of context each chunk of decode_chunked takes on either side."""
        return _lib.mh3a_decode_margin(self._h)

    def decode_chunked(self, latents, chunk_frames, flags=0, out=None, stream=None):
        """decode() in time chunks of chunk_frames latents, each decoded from
        a window widened by margin() latents per side and cropped; the
        workspace depends on chunk_frames, not on the sequence length."""
        torch = _torch()
        z = self._check_input(latents, 3, "latents")
        b, c, n = z.shape
        if c != self.latent_channels:
            raise ValueError(f"latents must have {self.latent_channels} channels")
        if out is None:
            out = torch.empty((b, 1, self.hop * n), dtype=torch.float32, device=z.device)
        nbytes = _lib.mh3a_decode_chunked_workspace_size(self._h, b, n, chunk_frames, flags)
        ws = self._workspace(nbytes)
        st = (stream or torch.cuda.current_stream(z.device)).cuda_stream
        _lib.mh3a_decode_chunked(self._h, z.data_ptr(), b, n, chunk_frames, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                 flags, st)
        return out

    def amp_stage(self, stage, x, flags=0, out=None, stream=None):
        torch = _torch()
        x = self._check_input(x, 3, "x")
        b, c, length = x.shape
        if out is None:
            out = torch.empty_like(x)
        nbytes = _lib.mh3a_amp_stage_workspace_size(self._h, stage, b, length)
        ws = self._workspace(nbytes)
        st = (stream or torch.cuda.current_stream(x.device)).cuda_stream
        _lib.mh3a_amp_stage(self._h, stage, x.data_ptr(), b, length, out.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                            st)
        return out


def to_numpy_params(params):
    return {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in params.items()}


class Encoder:
    """The encoder's convolution stack (waveform -> hidden), built once from
    host parameters (weight norm folded at construction)."""

    def __init__(self, params, config=None, device=0):
        self.config = dict(config or {})
        self.device = int(device)
        cfg = _lib.make_encoder_config(self.config)
        self.latent_dim = cfg.latent_dim
        self._h = _lib.mh3a_encoder_create(cfg, params, self.device)
        self._ws = None
        self._old_ws = []

    def close(self):
        if getattr(self, "_h", None):
            _lib.mh3a_encoder_destroy(self._h)
            self._h = None
        self._ws, self._old_ws = None, []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def frames(self, samples):
        return _lib.mh3a_encode_frames(self._h, samples)

    def workspace_size(self, batch, samples, flags=0):
        return _lib.mh3a_encode_workspace_size(self._h, batch, samples, flags)

    def encode_hidden(self, wave, flags=0, out=None, stream=None):
        torch = _torch()
        x = Decoder._check_input(wave, 3, "wave")
        b, c, s = x.shape
        if c != 1:
            raise ValueError("wave must be (B, 1, samples)")
        if out is None:
            out = torch.empty((b, self.latent_dim, self.frames(s)), dtype=torch.float32, device=x.device)
        nbytes = self.workspace_size(b, s, flags)
        if self._ws is None or self._ws.numel() < nbytes:
            if self._ws is not None:
                self._old_ws.append(self._ws)  # a captured graph may still use it
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=f"cuda:{self.device}")
        st = (stream or torch.cuda.current_stream(x.device)).cuda_stream
        _lib.mh3a_encode_hidden(self._h, x.data_ptr(), b, s, out.data_ptr(), self._ws.data_ptr(), self._ws.numel(),
                                flags, st)
        return out

    def timing(self, mode):
        _lib.mh3a_encoder_timing_enable(self._h, mode)

    def timing_read(self):
        return _lib.mh3a_encoder_timing_read(self._h)
