"""Oracle for the window/full-attention vision tower and its 2x2 patch merger.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg. Shares no code with the HIP path.

Source: Youtu-VL-4B ncnn port (ncnn discussion #6850), 实现流程 §3 and 结果展示:
27 vision layers; layers 7, 15, 23 and 26 attend globally, the others inside
windows of 8x8 merged patches; the window grouping is one row permutation
(window_index) and the mask is block-diagonal; 2D RoPE cos/sin and both masks
are runtime-built inputs; after post_layernorm the merger concatenates each
2x2 patch neighbourhood (1152*4 = 4608) and projects it with a two-layer MLP
to 2560. A 14x92 grid gives 1288 patches and 322 merged tokens. 2D RoPE: the
head is split in two halves, the first rotated by the row (h) position and the
second by the column (w) position (Penguin-VL ncnn port, ncnn discussion
#6868, §2.3).

Readings where the pages are silent (listed with the design notes):
  * pre-LayerNorm block (LN eps 1e-6 with shift), QKV/O/fc1/fc2 with biases,
    GELU in tanh form between fc1 and fc2 and between the two merger layers,
    no QK-Norm, softmax scale 1/sqrt(head_dim);
  * input rows arrive 2x2-group-major: rows 4u..4u+3 are the four patches of
    merge unit u, units in raster order of the merged grid, sub-patch order
    (0,0),(0,1),(1,0),(1,1);
  * windows tile the merged grid in window x window cells from the top-left;
    units are permuted window by window (windows in raster order, units in
    raster order inside each window); the merged output is returned in raster
    (unpermuted) unit order.
  * bf16 storage (the Mixed policy of the HunyuanOCR v1.5 port, §3.7: the
    vision tower keeps reduced-precision storage with fp32 accumulation; this
    library's reduced storage type is bf16): weights, biases and norm
    parameters hold bf16 values, the GEMM operands (normed rows, attention
    output, GELU output, merger operands) and q, k, v are rounded to bf16, the
    residual stream stays fp32 -- the same rounding points as the decoder,
    and the same exact (float64) sums of the exact bf16 products.
"""
import numpy as np

from .decoder import (BF16, BF16_F32SUM, BF16_MODES, MASK_NEG, _lin, bf16_round, gelu_tanh, layer_norm,
                      rope_apply, rope_tables, softmax_attention, F64)


def vit_window_order(cfg):
    """(unit permutation, window id per permuted unit).

    perm[p] = raster index of the merge unit placed at permuted slot p.
    """
    gh, gw = cfg.grid_h // cfg.merge, cfg.grid_w // cfg.merge
    win = cfg.window
    perm, seg = [], []
    wid = 0
    for wr in range(0, gh, win):
        for wc in range(0, gw, win):
            for r in range(wr, min(wr + win, gh)):
                for c in range(wc, min(wc + win, gw)):
                    perm.append(r * gw + c)
                    seg.append(wid)
            wid += 1
    return np.asarray(perm, np.int64), np.asarray(seg, np.int64)


def vit_positions(cfg):
    """(h, w) patch-grid position of every input row, shape [2, N]."""
    m = cfg.merge
    gw = cfg.grid_w // m
    r = np.arange(cfg.n_patches)
    u, sub = r // (m * m), r % (m * m)
    mr, mc = u // gw, u % gw
    return np.stack([m * mr + sub // m, m * mc + sub % m])


def vit_layer(x, w, mask_add, cos, sin, cfg, prec=F64):
    """Pre-LN ViT block over all rows (non-causal, additive mask)."""
    S = x.shape[0]
    nh, d = cfg.n_heads, cfg.head_dim
    h = layer_norm(x, w["attn_norm"], w["attn_norm_b"], cfg.eps)
    q = (_lin(h, w["wq"], prec) + w["bq"]).reshape(S, nh, d)
    k = (_lin(h, w["wk"], prec) + w["bk"]).reshape(S, nh, d)
    v = (_lin(h, w["wv"], prec) + w["bv"]).reshape(S, nh, d)
    q = rope_apply(q, cos, sin, 2)
    k = rope_apply(k, cos, sin, 2)
    if prec in BF16_MODES:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    o = softmax_attention(q.transpose(1, 0, 2), k.transpose(1, 0, 2), v.transpose(1, 0, 2), mask_add, 1)
    x = x + _lin(o.transpose(1, 0, 2).reshape(S, nh * d), w["wo"], prec) + w["bo"]
    h2 = layer_norm(x, w["mlp_norm"], w["mlp_norm_b"], cfg.eps)
    f = gelu_tanh(_lin(h2, w["w1"], prec) + w["b1"])
    return x + _lin(f, w["w2"], prec) + w["b2"]


def run_vit(cfg, glob, layers, prec=None):
    """Vision tower + merger. Returns out [n_merged, out_dim] in raster unit order,
    plus the permuted final hidden rows and the permutation. prec overrides the
    arithmetic mode (BF16_F32SUM only to measure the bf16 tower's noise floor)."""
    m2 = cfg.merge * cfg.merge
    perm_u, seg_u = vit_window_order(cfg)
    row_perm = (perm_u[:, None] * m2 + np.arange(m2)[None, :]).reshape(-1)
    seg_rows = np.repeat(seg_u, m2)
    x = np.asarray(glob["x"], np.float64)[row_perm]
    pos = vit_positions(cfg)[:, row_perm]
    half = cfg.head_dim // 2
    axes = np.concatenate([np.zeros(half // 2, np.int64), np.ones(half // 2, np.int64)])
    cos, sin = rope_tables(pos, axes, 2, cfg.head_dim, cfg.theta)
    win_mask = np.where(seg_rows[:, None] == seg_rows[None, :], 0.0, MASK_NEG)
    full_mask = np.zeros_like(win_mask)
    if prec is None:
        prec = BF16 if getattr(cfg, "dtype", "f32") == "bf16" else F64
    # matrices in the element type _lin contracts them in (bf16 values are exact in float64)
    mat = (lambda a: np.asarray(a, np.float32)) if prec == BF16_F32SUM else (lambda a: np.asarray(a, np.float64))
    ws = [{k: (mat(v) if v.ndim == 2 else np.asarray(v, np.float64)) for k, v in w.items()} for w in layers]
    for l, w in enumerate(ws):
        x = vit_layer(x, w, full_mask if l in cfg.full_layers else win_mask, cos, sin, cfg, prec)
    g = {k: (mat(v) if np.ndim(v) == 2 else np.asarray(v, np.float64)) for k, v in glob.items() if k != "x"}
    hpost = layer_norm(x, g["post_ln"], g["post_ln_b"], cfg.eps)
    z = hpost.reshape(cfg.n_merged, m2 * cfg.hidden)
    y = _lin(gelu_tanh(_lin(z, g["m1"], prec) + g["m1b"]), g["m2"], prec) + g["m2b"]
    out = np.empty_like(y)
    out[perm_u] = y
    return {"out": out, "x_final": x, "perm_units": perm_u, "seg_units": seg_u, "row_perm": row_perm}
