"""CPU oracle of the BigVGAN decode path -- test infrastructure only.

Only the test suite, the package's smoke check and the benchmark's CPU
baseline may import this package; the product path never does.
"""

from .mh3a_oracle import (  # noqa: F401
    DEFAULT_CONFIG,
    activation1d,
    amp_block,
    bessel_i0,
    causal_attention_heads_mean,
    conv1d,
    conv_transpose1d,
    decode,
    decode_item,
    decode_window,
    downsample2,
    encode,
    encode_hidden,
    encode_hidden_item,
    encode_item,
    fold_weight_norm,
    gelu,
    kaiser_beta,
    kaiser_sinc_filter,
    kaiser_window,
    pre_block_item,
    qkv_bias,
    receptive_radius_latents,
    snake,
    snake_beta,
    stage_amp,
    upsample2,
)
