"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds random draws and input dtype conversion only; none of the decoder's
arithmetic lives here.

Recipe (each tensor has its own stream):
  rng = numpy.random.default_rng(SeedSequence([config_id, tensor_id]))
  tensor_id = layer * 32 + slot for per-layer tensors, GLOBAL * 32 + slot otherwise.
  * Linear / embedding weights: 0.02 * N(0,1), drawn in float32.
  * Norm gains: 1 + 0.02 * N(0,1); LayerNorm shifts and biases: 0.02 * N(0,1).
  * Text ids: uniform on [0, V-1); the placeholder id is V-1, written at the
    image span only.
  * Image rows, hidden-state inputs and decode rows: N(0,1) float32.
  * bf16 workloads: every weight / gain / table value is rounded to bfloat16
    (round to nearest even) after the float32 draw; both sides see the same
    bf16 values, held here as float32 arrays.
"""
import numpy as np

from .configs import BF16, DecoderConfig, VitConfig

GLOBAL = 4096

# per-layer slots
S_ATTN_NORM, S_WQ, S_WK, S_WV, S_QNORM, S_KNORM, S_WO, S_MLP_NORM, S_WG, S_WU, S_WD = range(11)
S_ATTN_NORM_B, S_BQ, S_BK, S_BV, S_BO, S_MLP_NORM_B, S_B1, S_B2, S_FC1, S_FC2 = range(11, 21)
S_WQA, S_QANORM, S_WQB, S_WKVA, S_KVANORM, S_WKVB = range(21, 27)  # expanded MLA
# global slots
G_EMBED, G_FINAL_NORM, G_IDS, G_IMG, G_X, G_DECODE_X = range(6)
G_VIT_X, G_POST_LN, G_POST_LN_B, G_M1, G_M1B, G_M2, G_M2B = range(6, 13)


def _rng(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([config_id, tensor_id]))


def to_bf16_values(a: np.ndarray, inplace: bool = False) -> np.ndarray:
    """Round float32 input values to the nearest bfloat16 (ties to even).

    Input-dtype conversion of generated data; returns float32 arrays whose
    values are exactly representable in bfloat16. Finite inputs only (the
    generated data has no NaN/Inf); uint32 arithmetic cannot overflow for them.
    Works in place in fixed-size chunks so that large tables need no temporaries.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not inplace:
        a = a.copy()
    flat = a.reshape(-1).view(np.uint32)
    chunk = 1 << 20
    tmp = np.empty(min(chunk, flat.size), dtype=np.uint32)
    for i in range(0, flat.size, chunk):
        u = flat[i:i + chunk]
        t = tmp[:u.size]
        np.bitwise_and(u, np.uint32(0x7F800000), out=t)
        if (t == np.uint32(0x7F800000)).any():
            raise ValueError("to_bf16_values expects finite values")
        np.right_shift(u, np.uint32(16), out=t)
        np.bitwise_and(t, np.uint32(1), out=t)
        u += np.uint32(0x7FFF)
        u += t
        u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _normal(cfg_id, tid, shape, scale=1.0):
    x = _rng(cfg_id, tid).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _weight(cfg, tid, shape):
    w = _normal(cfg.config_id, tid, shape, 0.02)
    return to_bf16_values(w, inplace=True) if cfg.dtype == BF16 else w


def _gain(cfg, tid, n):
    g = np.float32(1.0) + _normal(cfg.config_id, tid, (n,), 0.02)
    return to_bf16_values(g, inplace=True) if cfg.dtype == BF16 else g


def _shift(cfg, tid, n):
    b = _normal(cfg.config_id, tid, (n,), 0.02)
    return to_bf16_values(b, inplace=True) if cfg.dtype == BF16 else b


def decoder_layer_weights(cfg: DecoderConfig, layer: int) -> dict:
    """Weights of one decoder layer, in the model's natural (unpacked) form.

    wq [nq*d, H], wk/wv [nkv*d, H], wo [H, nq*d], wg/wu [F, H], wd [H, F].
    """
    base = layer * 32
    H, d, F = cfg.hidden, cfg.head_dim, cfg.ffn
    if cfg.is_mla:
        # expanded MLA: wq_a [qr, H], q_a_norm [qr], wq_b [nq*d, qr], wkv_a [r + dr, H] (latent rows,
        # then the shared rotated-key rows), kv_a_norm [r], wkv_b [nq*(dn + dv), r] (per head: the dn
        # key rows, then the dv value rows), wo [H, nq*dv]
        nq, qr, r, dr, dv = cfg.n_q_heads, cfg.q_lora_rank, cfg.kv_lora_rank, cfg.qk_rope_dim, cfg.v_head_dim
        return {
            "attn_norm": _gain(cfg, base + S_ATTN_NORM, H),
            "wq_a": _weight(cfg, base + S_WQA, (qr, H)),
            "q_a_norm": _gain(cfg, base + S_QANORM, qr),
            "wq_b": _weight(cfg, base + S_WQB, (nq * d, qr)),
            "wkv_a": _weight(cfg, base + S_WKVA, (r + dr, H)),
            "kv_a_norm": _gain(cfg, base + S_KVANORM, r),
            "wkv_b": _weight(cfg, base + S_WKVB, (nq * (d - dr + dv), r)),
            "wo": _weight(cfg, base + S_WO, (H, nq * dv)),
            "mlp_norm": _gain(cfg, base + S_MLP_NORM, H),
            "wg": _weight(cfg, base + S_WG, (F, H)),
            "wu": _weight(cfg, base + S_WU, (F, H)),
            "wd": _weight(cfg, base + S_WD, (H, F)),
        }
    w = {
        "attn_norm": _gain(cfg, base + S_ATTN_NORM, H),
        "wq": _weight(cfg, base + S_WQ, (cfg.n_q_heads * d, H)),
        "wk": _weight(cfg, base + S_WK, (cfg.n_kv_heads * d, H)),
        "wv": _weight(cfg, base + S_WV, (cfg.n_kv_heads * d, H)),
        "wo": _weight(cfg, base + S_WO, (H, cfg.n_q_heads * d)),
        "mlp_norm": _gain(cfg, base + S_MLP_NORM, H),
        "wg": _weight(cfg, base + S_WG, (F, H)),
        "wu": _weight(cfg, base + S_WU, (F, H)),
        "wd": _weight(cfg, base + S_WD, (H, F)),
    }
    if cfg.qk_norm:
        w["q_norm"] = _gain(cfg, base + S_QNORM, d)
        w["k_norm"] = _gain(cfg, base + S_KNORM, d)
    return w


def decoder_globals(cfg: DecoderConfig) -> dict:
    """Embedding table, final norm, prompt ids, image rows and hidden inputs."""
    g = GLOBAL * 32
    out = {}
    if cfg.vocab > 0:
        out["embed"] = _weight(cfg, g + G_EMBED, (cfg.vocab, cfg.hidden))
        out["final_norm"] = _gain(cfg, g + G_FINAL_NORM, cfg.hidden)
        ids = _rng(cfg.config_id, g + G_IDS).integers(0, cfg.vocab - 1, size=cfg.seq, dtype=np.int64)
        ids = ids.astype(np.int32)
        ids[cfg.img_start:cfg.img_start + cfg.n_img] = cfg.placeholder_id
        out["ids"] = ids
        if cfg.n_img > 0:
            out["img"] = _normal(cfg.config_id, g + G_IMG, (cfg.n_img, cfg.hidden))
    else:
        out["x"] = _normal(cfg.config_id, g + G_X, (cfg.seq, cfg.hidden))
        out["decode_x"] = _normal(cfg.config_id, g + G_DECODE_X, (cfg.decode_steps, cfg.hidden))
    return out


def vit_layer_weights(cfg: VitConfig, layer: int) -> dict:
    """One pre-LayerNorm ViT layer: LN, QKV(+b), O(+b), LN, fc1(+b), fc2(+b)."""
    base = layer * 32
    H, F = cfg.hidden, cfg.ffn
    hd = cfg.n_heads * cfg.head_dim
    return {
        "attn_norm": _gain(cfg, base + S_ATTN_NORM, H),
        "attn_norm_b": _shift(cfg, base + S_ATTN_NORM_B, H),
        "wq": _weight(cfg, base + S_WQ, (hd, H)),
        "wk": _weight(cfg, base + S_WK, (hd, H)),
        "wv": _weight(cfg, base + S_WV, (hd, H)),
        "bq": _shift(cfg, base + S_BQ, hd),
        "bk": _shift(cfg, base + S_BK, hd),
        "bv": _shift(cfg, base + S_BV, hd),
        "wo": _weight(cfg, base + S_WO, (H, hd)),
        "bo": _shift(cfg, base + S_BO, H),
        "mlp_norm": _gain(cfg, base + S_MLP_NORM, H),
        "mlp_norm_b": _shift(cfg, base + S_MLP_NORM_B, H),
        "w1": _weight(cfg, base + S_FC1, (F, H)),
        "b1": _shift(cfg, base + S_B1, F),
        "w2": _weight(cfg, base + S_FC2, (H, F)),
        "b2": _shift(cfg, base + S_B2, H),
    }


def vit_globals(cfg: VitConfig) -> dict:
    """Patch-token input (rows in 2x2-group-major order) and merger weights."""
    g = GLOBAL * 32
    H4 = cfg.hidden * cfg.merge * cfg.merge
    return {
        "x": _normal(cfg.config_id, g + G_VIT_X, (cfg.n_patches, cfg.hidden)),
        "post_ln": _gain(cfg, g + G_POST_LN, cfg.hidden),
        "post_ln_b": _shift(cfg, g + G_POST_LN_B, cfg.hidden),
        "m1": _weight(cfg, g + G_M1, (cfg.merger_hidden, H4)),
        "m1b": _shift(cfg, g + G_M1B, cfg.merger_hidden),
        "m2": _weight(cfg, g + G_M2, (cfg.out_dim, cfg.merger_hidden)),
        "m2b": _shift(cfg, g + G_M2B, cfg.out_dim),
    }


def sampling_case(case_id: int, vocab: int, n_context: int, sigma: float = 3.0, n_draws: int = 1) -> dict:
    """Seeded sampler inputs: fp32 logits N(0, sigma^2) [vocab], context ids uniform on [0, vocab)
    [n_context] (repeats allowed), uniform draws u in [0, 1) [n_draws] (float32 values)."""
    rng = _rng(7000 + case_id, 0)
    logits = (rng.standard_normal(vocab, dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    ctx = rng.integers(0, vocab, size=n_context, dtype=np.int64).astype(np.int32)
    u = rng.random(n_draws, dtype=np.float32)
    return {"logits": logits, "context": ctx, "u": u}

