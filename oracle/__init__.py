"""CPU oracle for the VLM decoder hot path — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation of what the GPU path
computes: embedding lookup with image-row injection, the causal decoder stack
with its fixed-window KV cache, one-token decode, final RMSNorm, lm_head and
greedy argmax, plus the window/full-attention ViT tower with its 2x2 merger.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or run anything in this package. It shares no code with the HIP path
(decoder_prefill_decode_amd/); the only common dependency is vlm_synth, which
holds the seeded input generators and no arithmetic of the method.

Precision: fp32 workloads are evaluated in float64. bf16 workloads keep the
same bf16 values as the GPU path, round GEMM operands to bf16 at the points
the GPU does, and add the exact products of bf16 values in float64 (so no
summation order is built in); norm statistics, softmax and argmax are float64.

Parity status of each function is listed in the module docstrings; every
function here is pinned by a -m "not gpu" test in tests/test_oracle_pins.py.
"""
from .decoder import (MASK_NEG, bf16_round, decoder_layer, embed_inject, gelu_tanh, greedy_argmax,
                      layer_norm, lm_head_logits, rms_norm, rope_apply, rope_tables, run_decoder,
                      silu, softmax_attention, window_mask)
from .vit import run_vit, vit_layer, vit_positions, vit_window_order
