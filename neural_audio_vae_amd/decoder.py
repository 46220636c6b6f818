"""Decoder and Encoder: torch-tensor convenience over the mh3a C ABI.

torch supplies device memory and the stream; every step of the decode runs
in the library's HIP kernels. The C ABI takes raw device pointers and no
buffer sizes, so these wrappers check every tensor they hand to it (dtype,
device, contiguity and exact shape) before the call.
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


class _Workspaces:
    """One device workspace per stream (concurrent calls on different
    streams need distinct workspaces). A workspace is allocated on its own
    stream, so when a larger call outgrows it, freeing it is ordered after
    the kernels that used it. A workspace used while that stream was being
    captured into a HIP graph may still be referenced by the graph: such
    buffers are kept until close()."""

    def __init__(self, device):
        self.device = device
        self.by_stream = {}
        self.captured = []

    def get(self, nbytes, stream):
        torch = _torch()
        key = stream.cuda_stream
        ws = self.by_stream.get(key)
        capturing = torch.cuda.is_current_stream_capturing()
        if ws is None or ws.numel() < nbytes:
            if capturing:
                raise RuntimeError("the first call of a shape must run outside graph capture (it sizes the workspace)")
            with torch.cuda.stream(stream):
                ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=f"cuda:{self.device}")
            self.by_stream[key] = ws
        if capturing and not any(w is ws for w in self.captured):
            self.captured.append(ws)
        return ws

    def clear(self):
        self.by_stream, self.captured = {}, []


def _check_tensor(t, name, device, shape=None, ndim=None):
    """A float32, contiguous CUDA tensor on cuda:<device> (of `shape` if
    given); raises ValueError otherwise. Only reads the tensor's metadata."""
    import torch

    if not (getattr(t, "is_cuda", False) and getattr(t, "dtype", None) == torch.float32):
        raise ValueError(f"{name} must be a float32 CUDA tensor")
    if t.device.index != device:
        raise ValueError(f"{name} is on {t.device}, the library object on cuda:{device}")
    if ndim is not None and len(t.shape) != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _input(t, name, device, ndim, stream):
    """The input as a contiguous tensor; a temporary copy is marked as used
    by `stream` so that the allocator keeps it until the kernels are done."""
    _check_tensor(t, name, device, ndim=ndim)
    if t.is_contiguous():
        return t
    c = t.contiguous()
    c.record_stream(stream)
    return c


def _output(out, name, device, shape, stream):
    if out is None:
        torch = _torch()
        with torch.cuda.stream(stream):
            return torch.empty(shape, dtype=torch.float32, device=f"cuda:{device}")
    _check_tensor(out, name, device, shape=shape)
    if not out.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return out


def _stream(stream, device):
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream(device)


class Decoder:
    """A decoder built once from host parameters (weight norm folded and
    filters designed at construction).

    The decode only enqueues kernels on the given stream (no allocation,
    memset or synchronization inside the library), so a call can be
    captured into a HIP graph (torch.cuda.graph) once a first call of the
    same shape on that stream has sized its workspace."""

    def __init__(self, params, config=None, latents_mean=None, latents_std=None, device=0):
        self.config = dict(config or {})
        self.device = int(device)
        cfg = _lib.make_config(self.config)
        self.latent_channels = cfg.latent_channels
        self.hop = cfg.hop_length
        self.num_ups = cfg.num_ups
        self._h = _lib.mh3a_decoder_create(cfg, params, latents_mean, latents_std, self.device)
        self._ws = _Workspaces(self.device)

    def close(self):
        if getattr(self, "_h", None):
            _lib.mh3a_destroy(self._h)
            self._h = None
        if getattr(self, "_ws", None) is not None:
            self._ws.clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, batch, frames, flags=0):
        return _lib.mh3a_decode_workspace_size(self._h, batch, frames, flags)

    def _latents(self, latents, st):
        z = _input(latents, "latents", self.device, 3, st)
        if z.shape[1] != self.latent_channels:
            raise ValueError(f"latents must have {self.latent_channels} channels, got {z.shape[1]}")
        return z

    def decode(self, latents, flags=0, out=None, stream=None):
        st = _stream(stream, self.device)
        z = self._latents(latents, st)
        b, _, n = z.shape
        out = _output(out, "out", self.device, (b, 1, self.hop * n), st)
        ws = self._ws.get(self.workspace_size(b, n, flags), st)
        _lib.mh3a_decode(self._h, z.data_ptr(), b, n, out.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                         st.cuda_stream)
        return out

    def timing(self, enable):
        _lib.mh3a_timing_enable(self._h, enable)

    def timing_read(self):
        return _lib.mh3a_timing_read(self._h)

    def layer_shape(self, frames, upto):
        return _lib.mh3a_decode_layer_shape(self._h, frames, upto)

    def decode_partial(self, latents, upto, flags=0, stream=None):
        st = _stream(stream, self.device)
        z = self._latents(latents, st)
        b, _, n = z.shape
        ch, length = self.layer_shape(n, upto)
        out = _output(None, "out", self.device, (b, ch, length), st)
        ws = self._ws.get(self.workspace_size(b, n, flags), st)
        _lib.mh3a_decode_partial(self._h, z.data_ptr(), b, n, upto, out.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                                 st.cuda_stream)
        return out

    def margin(self):
        """Latents of context each chunk of decode_chunked takes on either side."""
        return _lib.mh3a_decode_margin(self._h)

    def decode_chunked(self, latents, chunk_frames, flags=0, out=None, stream=None):
        """decode() in time chunks of chunk_frames latents, each decoded from
        a window widened by margin() latents per side and cropped; the
        workspace depends on chunk_frames, not on the sequence length."""
        st = _stream(stream, self.device)
        z = self._latents(latents, st)
        b, _, n = z.shape
        out = _output(out, "out", self.device, (b, 1, self.hop * n), st)
        nbytes = _lib.mh3a_decode_chunked_workspace_size(self._h, b, n, chunk_frames, flags)
        ws = self._ws.get(nbytes, st)
        _lib.mh3a_decode_chunked(self._h, z.data_ptr(), b, n, chunk_frames, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                 flags, st.cuda_stream)
        return out

    def stage_channels(self, stage):
        """Channels of upsampling stage `stage` (its AMP set's width)."""
        if not 0 <= int(stage) < self.num_ups:
            raise ValueError(f"stage must be in [0, {self.num_ups})")
        return self.layer_shape(1, 3 + 2 * int(stage))[0]

    def amp_stage(self, stage, x, flags=0, out=None, stream=None):
        st = _stream(stream, self.device)
        x = _input(x, "x", self.device, 3, st)
        b, c, length = x.shape
        if c != self.stage_channels(stage):
            raise ValueError(f"stage {stage} has {self.stage_channels(stage)} channels, x has {c}")
        out = _output(out, "out", self.device, (b, c, length), st)
        nbytes = _lib.mh3a_amp_stage_workspace_size(self._h, stage, b, length)
        ws = self._ws.get(nbytes, st)
        _lib.mh3a_amp_stage(self._h, stage, x.data_ptr(), b, length, out.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                            st.cuda_stream)
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
        self.latent_channels = cfg.latent_channels
        self._h = _lib.mh3a_encoder_create(cfg, params, self.device)
        self._ws = _Workspaces(self.device)

    def close(self):
        if getattr(self, "_h", None):
            _lib.mh3a_encoder_destroy(self._h)
            self._h = None
        if getattr(self, "_ws", None) is not None:
            self._ws.clear()

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
        st = _stream(stream, self.device)
        x = _input(wave, "wave", self.device, 3, st)
        b, c, s = x.shape
        if c != 1:
            raise ValueError("wave must be (B, 1, samples)")
        out = _output(out, "out", self.device, (b, self.latent_dim, self.frames(s)), st)
        ws = self._ws.get(self.workspace_size(b, s, flags), st)
        _lib.mh3a_encode_hidden(self._h, x.data_ptr(), b, s, out.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                                st.cuda_stream)
        return out

    def encode_mean(self, wave, flags=0, out=None, stream=None):
        """Waveform (B, 1, S) -> posterior mean (B, latent_channels,
        ceil(S / hop)): the convolution stack, the attention projection and
        mean_proj (the encoder must hold the pre_block parameters)."""
        st = _stream(stream, self.device)
        x = _input(wave, "wave", self.device, 3, st)
        b, c, s = x.shape
        if c != 1:
            raise ValueError("wave must be (B, 1, samples)")
        out = _output(out, "out", self.device, (b, self.latent_channels, self.frames(s)), st)
        ws = self._ws.get(_lib.mh3a_encode_mean_workspace_size(self._h, b, s, flags), st)
        _lib.mh3a_encode_mean(self._h, x.data_ptr(), b, s, out.data_ptr(), ws.data_ptr(), ws.numel(), flags,
                              st.cuda_stream)
        return out

    def timing(self, mode):
        _lib.mh3a_encoder_timing_enable(self._h, mode)

    def timing_read(self):
        return _lib.mh3a_encoder_timing_read(self._h)
