"""CPU oracle for group-wise asymmetric INT4 weight quantization, the W4A16
linear layer and the activation-aware scale search.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this package. It shares no code with the HIP library and
imports nothing from it.
"""

from .awq_oracle import (  # noqa: F401
    QMAX,
    RANGE_FLOOR,
    MEAN_FLOOR,
    SYM_QMAX,
    SYM_ZERO,
    group_quantize,
    group_quantize_symmetric,
    quantize_symmetric,
    clip_position,
    clip_bounds,
    group_quantize_clipped,
    quantize_clipped,
    clipped_weight,
    clip_search,
    pack_codes,
    unpack_codes,
    quantize,
    dequantize,
    linear_ref,
    activation_absmean,
    alpha_grid,
    channel_scales,
    searched_weight,
    search_loss_direct,
    scaled_activations_f16,
    search_loss_f16_activations,
    gram,
    search_loss_gram,
    scale_search,
    salient_count,
    salient_channels,
    mixed_weight,
    quantize_salient,
    dequantize_salient,
    linear_salient_ref,
    salient_loss,
    group_quantize_bits,
    pack_codes8,
    unpack_codes8,
    quantize_w8,
    dequantize_w8,
    linear_ref_w8,
)
