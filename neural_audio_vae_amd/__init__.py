"""mh3a: the MiniMax-H3 audio-VAE BigVGAN decoder as hand-written gfx950
HIP kernels behind a C ABI (include/mh3a.h).

    from neural_audio_vae_amd import Decoder
    dec = Decoder(params)            # dict name -> float32 array
    wave = dec.decode(latents)       # (B, 32, N) cuda fp32 -> (B, 1, 800 N)

    from neural_audio_vae_amd import Encoder
    enc = Encoder(enc_params)        # the encoder's convolution stack
    hidden = enc.encode_hidden(wave) # (B, 1, S) -> (B, 2048, ceil(S / 800))

Importing the package does not load the library; constructing a Decoder
does, and fails if libmh3a.so has not been built.
"""

from ._lib import (MH3A_FLAG_BATCH_INVARIANT, MH3A_FLAG_BF16_MFMA, MH3A_FLAG_DENORMALIZE,  # noqa: F401
                   MH3A_FLAG_NO_CLAMP, MH3AError)  # noqa: F401
from .decoder import Decoder, Encoder  # noqa: F401
