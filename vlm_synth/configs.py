"""Workload shapes for the five synthetic decoder / vision configurations.

This module only names sizes. It holds none of the decoder arithmetic, so both
the CPU oracle and the GPU path may import it.

Shape origins (cited by page title and section):
  * 512-token fixed window, 322 merged visual tokens from a 14x92 patch grid:
    Youtu-VL-4B ncnn port (ncnn discussion #6850), 结果展示 and 实现流程 §7.
  * Qwen3 language model: hidden 1024, 28 layers, 16 query / 8 KV heads,
    head_dim 128, vocab 151936, tied embedding, theta 1e6, eps 1e-6;
    495 = 9x55 image patches: Penguin-VL ncnn port (ncnn discussion #6868),
    §2.1 and §2.3.
  * 27-layer window/full-attention vision tower with 2x2 merge to 2560:
    Youtu-VL-4B ncnn port, 实现流程 §3.
Unstated values (KV window of the tiny and 28-layer stacks, image span start,
placeholder id) are readings documented with the design notes.
"""
from dataclasses import dataclass, field
from typing import Tuple

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class DecoderConfig:
    name: str
    config_id: int          # seed stream selector
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int              # 0: no embedding table / lm_head (hidden-state workload)
    seq: int                # prefill length S
    n_img: int              # injected image rows (0: none)
    img_start: int          # first placeholder row
    decode_steps: int
    capacity: int           # KV window W (slots)
    dtype: str              # f32 or bf16 (weights, KV cache, GEMM operands)
    qk_norm: int            # 0 off, 1 per-head q/k RMSNorm before RoPE, 2 after RoPE
    theta: float = 1.0e6
    eps: float = 1.0e-6
    rope_interleave: bool = False  # RoPE pairs adjacent elements (de-interleaved before rotate-half)
    # multi-head latent attention, expanded per head (kv_lora_rank > 0): head_dim is the q/k head width,
    # qk_nope_dim + qk_rope_dim; v_head_dim the value width; only the qk_rope_dim part rotates
    q_lora_rank: int = 0
    kv_lora_rank: int = 0
    qk_rope_dim: int = 0
    v_head_dim: int = 0

    @property
    def is_mla(self) -> bool:
        return self.kv_lora_rank > 0

    @property
    def v_dim(self) -> int:
        return self.v_head_dim if self.is_mla else self.head_dim

    @property
    def rope_dim(self) -> int:
        return self.qk_rope_dim if self.is_mla else self.head_dim

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def placeholder_id(self) -> int:
        return self.vocab - 1


@dataclass(frozen=True)
class VitConfig:
    name: str
    config_id: int
    n_layers: int
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    grid_h: int             # raw patch grid
    grid_w: int
    merge: int              # 2x2 merge
    window: int             # window side in merged cells
    full_layers: Tuple[int, ...]
    merger_hidden: int
    out_dim: int
    dtype: str = F32
    theta: float = 1.0e6
    eps: float = 1.0e-6

    @property
    def n_patches(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def n_merged(self) -> int:
        return self.n_patches // (self.merge * self.merge)

    @property
    def qkv_rows(self) -> int:
        return 3 * self.n_heads * self.head_dim


C1 = DecoderConfig("c1_tiny", 1, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2,
                   head_dim=64, ffn=768, vocab=4096, seq=32, n_img=16, img_start=8,
                   decode_steps=8, capacity=64, dtype=F32, qk_norm=False)

C2_F32 = DecoderConfig("c2_layer_f32", 2, n_layers=1, hidden=1024, n_q_heads=16, n_kv_heads=8,
                       head_dim=128, ffn=3072, vocab=0, seq=512, n_img=0, img_start=0,
                       decode_steps=64, capacity=1024, dtype=F32, qk_norm=True)

C2_BF16 = DecoderConfig("c2_layer_bf16", 2, n_layers=1, hidden=1024, n_q_heads=16, n_kv_heads=8,
                        head_dim=128, ffn=3072, vocab=0, seq=512, n_img=0, img_start=0,
                        decode_steps=64, capacity=1024, dtype=BF16, qk_norm=True)

C3 = DecoderConfig("c3_qwen3_28l", 3, n_layers=28, hidden=1024, n_q_heads=16, n_kv_heads=8,
                   head_dim=128, ffn=3072, vocab=151936, seq=560, n_img=495, img_start=32,
                   decode_steps=128, capacity=1024, dtype=BF16, qk_norm=True)

C4 = DecoderConfig("c4_llama_4b", 4, n_layers=36, hidden=2560, n_q_heads=32, n_kv_heads=8,
                   head_dim=80, ffn=9728, vocab=128256, seq=512, n_img=322, img_start=32,
                   decode_steps=256, capacity=2048, dtype=BF16, qk_norm=False)

C5 = VitConfig("c5_vit_27l", 5, n_layers=27, hidden=1152, n_heads=16, head_dim=72, ffn=4304,
               grid_h=14, grid_w=92, merge=2, window=8, full_layers=(7, 15, 23, 26),
               merger_hidden=4608, out_dim=2560)

# Youtu-LLM-style expanded MLA layer stack at reduced width (the pages: 32 heads, K 192 = 128 + 64
# rotated, V 128, 512-wide latent, interleaved RoPE); q_lora_rank is a reading (the pages give none).
C_MLA = DecoderConfig("c_mla_small", 6, n_layers=2, hidden=512, n_q_heads=4, n_kv_heads=4, head_dim=192,
                      ffn=1024, vocab=4096, seq=48, n_img=12, img_start=8, decode_steps=8, capacity=128,
                      dtype=F32, qk_norm=0, rope_interleave=True, q_lora_rank=384, kv_lora_rank=512,
                      qk_rope_dim=64, v_head_dim=128)

DECODER_CONFIGS = {c.name: c for c in (C1, C2_F32, C2_BF16, C3, C4)}
ALL_CONFIGS = dict(DECODER_CONFIGS, **{C5.name: C5})


def scaled(cfg: DecoderConfig, **over) -> DecoderConfig:
    """A copy of cfg with some sizes replaced (for small parity cases)."""
    d = dict(cfg.__dict__)
    d.update(over)
    return DecoderConfig(**d)


def scaled_vit(cfg: VitConfig, **over) -> VitConfig:
    d = dict(cfg.__dict__)
    d.update(over)
    return VitConfig(**d)
