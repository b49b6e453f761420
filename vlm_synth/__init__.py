"""Seeded synthetic workloads (shapes and random inputs only)."""
from .configs import (ALL_CONFIGS, BF16, C1, C2_BF16, C2_F32, C3, C4, C5, C_MLA, DECODER_CONFIGS, F32,
                      DecoderConfig, VitConfig, scaled, scaled_vit)
from .gen import (bf16_bits, decoder_globals, decoder_layer_weights, sampling_case, to_bf16_values, vit_globals,
                  vit_layer_weights)
