"""Oracle for the decoder stack: prefill, fixed-window KV cache, decode, head.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg. Shares no code with the HIP path.

Sources (page title, section):
  [Youtu]   Youtu-VL-4B ncnn port (ncnn discussion #6850)
  [Penguin] Penguin-VL ncnn port (ncnn discussion #6868)
  [HyOCR15] HunyuanOCR v1.5 ncnn port, technical report (ncnn discussion #6846)
  [HyOCR10] HunyuanOCR v1.0 ncnn port (ncnn discussion #6847)

What the pages fix, in the order this file follows it:
  * Text rows come from a lookup in the (tied) embedding table; rows whose id
    is the image placeholder are overwritten, in order, by the projector rows,
    and the placeholder count must equal the number of projector rows
    ([Youtu] 实现流程 §5; [HyOCR15] §3.2).
  * Each decoder layer takes (x, cos, sin, mask) and returns hidden states
    plus the K/V it adds to the cache ([Youtu] 实现流程 §6; [HyOCR10] 四.3).
  * Qwen3 layer order: input RMSNorm, q/k/v projections, per-head q/k RMSNorm,
    rotate-half RoPE, GQA attention, o-projection with residual, post RMSNorm,
    SwiGLU MLP with residual ([Penguin] §2.1, §4.2, §5.4). GQA: KV head j
    serves the query heads that the export expands it to with
    repeat_interleave, i.e. query head h reads KV head h // (nq / nkv)
    ([Penguin] §3).
  * RoPE is q*cos + rotate_half(q)*sin with cos/sin fed from outside
    ([Youtu] 实现难点 §2, 实现流程 §6); the interleaved variant de-interleaves
    the head first ([Youtu] 实现难点 §2). HunyuanOCR applies the per-head
    q/k RMSNorm after RoPE instead of before, and the cache stores the
    normalised k ([HyOCR10] 二, 五.2). Its multi-axis RoPE base is
    theta * alpha^(d/(d-2)) ([HyOCR10] 五.1).
  * Softmax is written out as max, subtract, exp, sum, divide ([Youtu] 实现难点 §3).
  * The KV cache is a fixed window per layer; a finite additive mask holds 0
    for valid slots (position <= t) and -1e9 elsewhere; the runtime writes the
    current token's K/V into slot t ([Youtu] 实现流程 §7; [HyOCR10] 五.6).
  * After prefill the first token is the greedy argmax of the logits of the
    last real row; each decode step embeds the previous token, runs every
    layer against the cache, applies the final RMSNorm and the lm_head (a dot
    product with every row of the tied table) and takes the argmax
    ([Youtu] 实现流程 §6, §8, 解码与采样说明; [HyOCR15] §3.4).

Readings where the pages are silent (listed with the design notes):
  argmax ties go to the lowest index; non-finite logits are an error; theta
  is 1e6; RMSNorm eps 1e-6; in bf16 mode the GEMM A-operands (normed rows,
  attention output, SwiGLU product, final-norm row), q and the cached k/v are
  rounded to bf16 (ties to even), the softmax P stays unrounded.
  bf16 storage with fp32 accumulation (the Mixed policy of [HyOCR15] §3.7)
  is read as: the products of bf16 values are exact, and the oracle adds them
  exactly (float64 sums of the float64 products), so its result does not
  depend on a summation order. BF16_F32SUM keeps every operand and rounding
  point but sums in float32 BLAS order; it exists only to measure how far a
  valid float32 summation order moves the results (the noise floor that
  decides which greedy steps are near-ties).
"""
import time

import numpy as np

MASK_NEG = -1.0e9          # finite "minus infinity" of the fixed-window mask
QK_NORM_BEFORE_ROPE = 1    # Qwen3 order ([Penguin] §5.4)
QK_NORM_AFTER_ROPE = 2     # HunyuanOCR order: the cache holds the normalised k ([HyOCR10] 五.2)
F64 = "f64"
BF16 = "bf16"                # bf16 operands and rounding points, exact (float64) sums
BF16_F32SUM = "bf16_f32sum"  # the same, summed in float32 BLAS order (noise-floor measurement only)
BF16_MODES = (BF16, BF16_F32SUM)


# ----------------------------------------------------------------------------
# scalar building blocks
# ----------------------------------------------------------------------------
def bf16_round(a):
    """Nearest bfloat16 value (8 significant bits, ties to even), as float64.

    Written from the format definition: a = m * 2**e with 0.5 <= |m| < 1, keep
    8 significant bits of m with round-half-even. Values beyond the bf16 range
    become +-inf. (Subnormal bf16 values are not produced by these workloads.)
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    m = np.rint(m * 256.0) / 256.0
    out = np.ldexp(m, e)
    big = np.abs(out) >= 2.0 ** 128
    if np.any(big):
        out = np.where(big, np.copysign(np.inf, out), out)
    return out


def rms_norm(x, gain, eps):
    """x / sqrt(mean(x^2) + eps) * gain over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def layer_norm(x, gain, shift, eps):
    """(x - mean) / sqrt(var + eps) * gain + shift over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1, keepdims=True)
    xc = x - mu
    var = np.mean(xc * xc, axis=-1, keepdims=True)
    return xc / np.sqrt(var + eps) * np.asarray(gain, np.float64) + np.asarray(shift, np.float64)


def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z):
    """GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def _lin(a, w, prec):
    """a @ w.T.

    F64: float64. BF16: a rounded to bf16; w holds bf16 values as float64, so
    every product is exact and the float64 sums are exact to ~1e-16 relative.
    BF16_F32SUM: the same operands summed by float32 BLAS (w float32)."""
    if prec == BF16:
        return bf16_round(a) @ np.asarray(w, np.float64).T
    if prec == BF16_F32SUM:
        ar = bf16_round(a).astype(np.float32)
        return (ar @ np.asarray(w, np.float32).T).astype(np.float64)
    return np.asarray(a, np.float64) @ w.T


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------
def rope_tables(positions, axis_of_pair, n_seg, head_dim, theta):
    """cos/sin tables [T, head_dim] for rotate-half RoPE, float64.

    positions: int array [n_axes, T] (text: one axis 0..T-1; 2D vision: h and w;
    multi-axis xdRoPE/mRoPE: one row per axis). The head is split into n_seg
    rotation segments of length d_seg = head_dim / n_seg; within a segment,
    pair j (element j with element j + d_seg/2) turns at inv_freq_j =
    theta^(-2j/d_seg) times the position of axis axis_of_pair[seg*d_seg/2 + j].
    Two segments with axes (h, w) is the 2D vision RoPE of [Penguin] §2.3
    (first half of the head from the h stream, second half from the w stream);
    one segment with per-pair axes is the multi-axis form of [HyOCR15] §3.3.
    """
    positions = np.atleast_2d(np.asarray(positions, dtype=np.int64))
    T = positions.shape[1]
    seg = head_dim // n_seg
    half = seg // 2
    assert seg * n_seg == head_dim and half * 2 == seg
    axis_of_pair = np.asarray(axis_of_pair, dtype=np.int64)
    assert axis_of_pair.shape == (head_dim // 2,)
    cos = np.empty((T, head_dim), dtype=np.float64)
    sin = np.empty((T, head_dim), dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / seg)
    for s in range(n_seg):
        for j in range(half):
            ang = positions[axis_of_pair[s * half + j]].astype(np.float64) * inv_freq[j]
            c, sn = np.cos(ang), np.sin(ang)
            cos[:, s * seg + j] = c
            cos[:, s * seg + j + half] = c
            sin[:, s * seg + j] = sn
            sin[:, s * seg + j + half] = sn
    return cos, sin


def deinterleave(u, n_seg):
    """Per segment, the even-indexed elements, then the odd-indexed ones.

    The interleaved RoPE of [Youtu] 实现难点 §2 views each head as d/2 adjacent
    pairs and transposes that view before rotate-half: adjacent elements
    (2i, 2i+1) become elements (i, i + d/2), the pair that rotate-half turns
    together. Output stays in this de-interleaved order (it is what the cache
    holds); q and k share it, so q.k is unchanged by the reordering itself.
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    seg = d // n_seg
    out = np.empty_like(u)
    for s in range(n_seg):
        part = u[..., s * seg:(s + 1) * seg]
        out[..., s * seg:(s + 1) * seg] = np.concatenate([part[..., 0::2], part[..., 1::2]], axis=-1)
    return out


def alpha_scaled_base(theta, alpha, head_dim):
    """Effective RoPE base theta * alpha^(d / (d - 2)) ([HyOCR10] 五.1)."""
    d = float(head_dim)
    return float(theta) * float(alpha) ** (d / (d - 2.0))


def rope_apply(u, cos, sin, n_seg, interleave=False):
    """u*cos + rotate_half(u)*sin per segment; rotate_half(a, b) = (-b, a).

    u: [T, heads, d]; cos/sin: [T, d]. interleave: de-interleave u first
    (deinterleave above), the interleaved form of [Youtu] 实现难点 §2.
    """
    u = deinterleave(u, n_seg) if interleave else np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    seg = d // n_seg
    half = seg // 2
    rot = np.empty_like(u)
    for s in range(n_seg):
        a = u[..., s * seg: s * seg + half]
        b = u[..., s * seg + half: (s + 1) * seg]
        rot[..., s * seg: s * seg + half] = -b
        rot[..., s * seg + half: (s + 1) * seg] = a
    return u * cos[:, None, :] + rot * sin[:, None, :]


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def window_mask(S, pos0, W):
    """Additive fixed-window mask [S, W]: 0 where slot j <= pos0 + s, else -1e9."""
    j = np.arange(W)[None, :]
    t = pos0 + np.arange(S)[:, None]
    return np.where(j <= t, 0.0, MASK_NEG)


def softmax_attention(q, k, v, mask_add, group):
    """Scaled dot-product attention with an additive mask, written out.

    q [nq, Sq, d]; k, v [nkv, Sk, d]; mask_add [Sq, Sk]; query head h reads KV
    head h // group. Softmax steps: max, subtract, exp, sum, divide.
    """
    nq, Sq, d = q.shape
    out = np.empty((nq, Sq, v.shape[-1]), dtype=np.float64)
    scale = 1.0 / np.sqrt(d)
    for h in range(nq):
        g = h // group
        s = (q[h] @ k[g].T) * scale + mask_add
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[h] = p @ v[g]
    return out


# ----------------------------------------------------------------------------
# embedding / injection
# ----------------------------------------------------------------------------
def embed_inject(embed, ids, placeholder_id, img):
    """x = E[ids]; placeholder rows replaced in order by img rows (count checked)."""
    x = np.asarray(embed, dtype=np.float64)[np.asarray(ids)]
    pos = np.nonzero(np.asarray(ids) == placeholder_id)[0]
    n_img = 0 if img is None else len(img)
    if len(pos) != n_img:
        raise ValueError(f"placeholder count {len(pos)} != image rows {n_img}")
    if n_img:
        x[pos] = np.asarray(img, dtype=np.float64)
    return x


# ----------------------------------------------------------------------------
# decoder layer
# ----------------------------------------------------------------------------
def decoder_layer(x, w, cfg, k_cache, v_cache, pos0, cos, sin, prec):
    """One Qwen3/Llama-style layer over rows pos0..pos0+S-1 (in place on caches).

    x: [S, H] float64. w: natural-form weights (wq, wk, wv, wo, wg, wu, wd,
    attn_norm, mlp_norm, optional q_norm/k_norm); in f64 mode float64 arrays,
    in bf16 mode float32 arrays of bf16 values. k_cache, v_cache: [nkv, W, d]
    float64 (bf16 values in bf16 mode). cos/sin: [>= pos0+S, d].
    Returns the new x.
    """
    S = x.shape[0]
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    W = k_cache.shape[1]
    if pos0 + S > W:
        raise ValueError("sequence exceeds the KV window")
    h = rms_norm(x, w["attn_norm"], cfg.eps)
    q = _lin(h, w["wq"], prec).reshape(S, nq, d)
    k = _lin(h, w["wk"], prec).reshape(S, nkv, d)
    v = _lin(h, w["wv"], prec).reshape(S, nkv, d)
    qkn = int(cfg.qk_norm)
    ilv = bool(getattr(cfg, "rope_interleave", False))
    if qkn == QK_NORM_BEFORE_ROPE:
        q = rms_norm(q, w["q_norm"], cfg.eps)
        k = rms_norm(k, w["k_norm"], cfg.eps)
    c, s_ = cos[pos0:pos0 + S], sin[pos0:pos0 + S]
    q = rope_apply(q, c, s_, 1, ilv)
    k = rope_apply(k, c, s_, 1, ilv)
    if qkn == QK_NORM_AFTER_ROPE:
        q = rms_norm(q, w["q_norm"], cfg.eps)
        k = rms_norm(k, w["k_norm"], cfg.eps)
    if prec in BF16_MODES:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    k_cache[:, pos0:pos0 + S] = k.transpose(1, 0, 2)
    v_cache[:, pos0:pos0 + S] = v.transpose(1, 0, 2)
    o = softmax_attention(q.transpose(1, 0, 2), k_cache, v_cache, window_mask(S, pos0, W), nq // nkv)
    o = o.transpose(1, 0, 2).reshape(S, nq * d)
    x = x + _lin(o, w["wo"], prec)
    return _mlp(x, w, cfg, prec)


def _mlp(x, w, cfg, prec):
    """Post-attention RMSNorm, SwiGLU MLP and residual ([Penguin] §2.1, §4.2)."""
    h2 = rms_norm(x, w["mlp_norm"], cfg.eps)
    a = silu(_lin(h2, w["wg"], prec)) * _lin(h2, w["wu"], prec)
    return x + _lin(a, w["wd"], prec)


def mla_layer(x, w, cfg, k_cache, v_cache, pos0, cos, sin, prec):
    """One multi-head latent attention layer in the expanded form ([Youtu] 实现流程 §6).

    The page's port does not absorb the latent: kv_b expands the 512-wide
    compressed KV into full per-head keys and values, the cache holds those
    (keys dn + dr wide, values dv wide), and every query head has its own KV
    head; the q and kv paths each have a low-rank a/b projection pair. The
    rotated part of the keys is the dr-wide tail of the kv_a output, shared by
    all heads; RoPE is interleaved on the dr-wide parts ([Youtu] 实现难点 §2,
    the 64x64 permutation). Order (the pages name the pieces, not the order;
    this is the plainest arrangement of them):
      h = RMSNorm(x)
      q = RMSNorm(h Wq_a^T) Wq_b^T, per head [q_nope (dn) | q_rope (dr)]
      [c (r) | k_rope (dr)] = h Wkv_a^T;  per head [k_nope (dn) | v (dv)] = RMSNorm(c) Wkv_b^T
      q = [q_nope | RoPE(q_rope)], k = [k_nope | RoPE(k_rope)]   (the shared k_rope in every head)
      attention with scale 1 / sqrt(dn + dr), o Wo^T added to x, then the SwiGLU MLP.
    k_cache [nq, W, dn + dr], v_cache [nq, W, dv]; cos/sin: [>= pos0+S, dr] tables.
    """
    S = x.shape[0]
    nq, d, dr, dv, r = cfg.n_q_heads, cfg.head_dim, cfg.qk_rope_dim, cfg.v_head_dim, cfg.kv_lora_rank
    dn = d - dr
    W = k_cache.shape[1]
    if pos0 + S > W:
        raise ValueError("sequence exceeds the KV window")
    ilv = bool(cfg.rope_interleave)
    h = rms_norm(x, w["attn_norm"], cfg.eps)
    qa = rms_norm(_lin(h, w["wq_a"], prec), w["q_a_norm"], cfg.eps)
    q = _lin(qa, w["wq_b"], prec).reshape(S, nq, d)
    ckv = _lin(h, w["wkv_a"], prec)
    c = rms_norm(ckv[:, :r], w["kv_a_norm"], cfg.eps)
    kv = _lin(c, w["wkv_b"], prec).reshape(S, nq, dn + dv)
    cr, sr = cos[pos0:pos0 + S], sin[pos0:pos0 + S]
    q_rope = rope_apply(q[..., dn:], cr, sr, 1, ilv)
    k_rope = rope_apply(ckv[:, None, r:], cr, sr, 1, ilv)
    q = np.concatenate([q[..., :dn], q_rope], axis=-1)
    k = np.concatenate([kv[..., :dn], np.broadcast_to(k_rope, (S, nq, dr))], axis=-1)
    v = kv[..., dn:]
    if prec in BF16_MODES:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    k_cache[:, pos0:pos0 + S] = k.transpose(1, 0, 2)
    v_cache[:, pos0:pos0 + S] = v.transpose(1, 0, 2)
    o = softmax_attention(q.transpose(1, 0, 2), k_cache, v_cache, window_mask(S, pos0, W), 1)
    o = o.transpose(1, 0, 2).reshape(S, nq * dv)
    x = x + _lin(o, w["wo"], prec)
    return _mlp(x, w, cfg, prec)


# ----------------------------------------------------------------------------
# head
# ----------------------------------------------------------------------------
def lm_head_logits(x_row, gain, table, eps, prec):
    """Final RMSNorm of one row, then its dot product with every table row."""
    hf = rms_norm(np.asarray(x_row, np.float64)[None, :], gain, eps)
    return _lin(hf, table, prec)[0]


def greedy_argmax(logits):
    """Index of the largest logit, lowest index on ties; non-finite is an error."""
    logits = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(logits)):
        raise FloatingPointError("non-finite logits")
    return int(np.argmax(logits))


def _top2_margin(logits):
    part = np.partition(np.asarray(logits, np.float64), -2)
    return float(part[-1] - part[-2])


# ----------------------------------------------------------------------------
# whole run
# ----------------------------------------------------------------------------
def _prep_weights(w, prec):
    if prec == BF16_F32SUM:
        return {k: np.asarray(v, dtype=np.float32) for k, v in w.items()}
    return {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}


def run_decoder(cfg, glob, layers, steps=None, prefill_split=None, keep_logits=False, sampler=None,
                prec=None, forced_ids=None):
    """Prefill the prompt, then greedy-decode `steps` tokens (default cfg.decode_steps).

    glob: vlm_synth.decoder_globals(cfg); layers: list of decoder_layer_weights.
    prefill_split: optional t0 < S; prefill only rows [0, t0) in parallel and
      feed rows t0..S-1 one at a time through the decode path (replay).
    sampler: optional f(logits, context_ids, i) -> id replacing the greedy argmax
      of the i-th generated token; context_ids are the prompt ids and the ids
      generated so far (oracle/sampling.py provides the sampler itself).
    prec: override of the arithmetic mode (default F64 for f32 workloads, BF16
      for bf16 ones; BF16_F32SUM only to measure the noise floor).
    forced_ids: teacher forcing; decode step i embeds forced_ids[i] instead of
      the previous pick (ids, margins and logits are still the stack's own).
    layers may be any sequence; each element is read once, so a lazy sequence
      keeps only one layer's input arrays alive at a time.
    Returns a dict with x_in [S,H], prefill_x [S,H] (hidden after the stack),
    k_cache/v_cache [L,nkv,W,d], logits0 (head of the last prompt row, vocab>0),
    ids [steps+1], margins [steps+1], decode_x [steps,H] (hidden after the
    stack for each decode step).
    """
    if prec is None:
        prec = BF16 if cfg.dtype == "bf16" else F64
    steps = cfg.decode_steps if steps is None else steps
    L, W = cfg.n_layers, cfg.capacity
    ws = [_prep_weights(w, prec) for w in layers]
    assert len(ws) == L
    mla = getattr(cfg, "kv_lora_rank", 0) > 0
    rd = cfg.qk_rope_dim if mla else cfg.head_dim   # width of the rotated part of a head
    cos, sin = rope_tables(np.arange(W)[None, :], np.zeros(rd // 2, np.int64), 1, rd, cfg.theta)
    kc = np.zeros((L, cfg.n_kv_heads, W, cfg.head_dim))
    vc = np.zeros((L, cfg.n_kv_heads, W, cfg.v_head_dim if mla else cfg.head_dim))
    layer_fn = mla_layer if mla else decoder_layer
    has_vocab = cfg.vocab > 0
    if has_vocab:
        table = np.asarray(glob["embed"], np.float32 if prec == BF16_F32SUM else np.float64)
        x = embed_inject(glob["embed"], glob["ids"], cfg.placeholder_id, glob.get("img"))
    else:
        x = np.asarray(glob["x"], np.float64)
    x_in = x.copy()
    S = x.shape[0]

    def stack(rows, pos0):
        for l in range(L):
            rows = layer_fn(rows, ws[l], cfg, kc[l], vc[l], pos0, cos, sin, prec)
        return rows

    t_start = time.perf_counter()
    t0 = S if prefill_split is None else prefill_split
    out = stack(x, 0) if t0 == S else stack(x[:t0], 0)
    if t0 < S:
        rows = [out]
        for t in range(t0, S):
            rows.append(stack(x[t:t + 1], t))
        out = np.concatenate(rows, axis=0)
    res = {"x_in": x_in, "prefill_x": out, "k_cache": kc, "v_cache": vc}
    ids, margins, dec_x, all_logits = [], [], [], []
    prompt_ids = [int(i) for i in np.asarray(glob["ids"])] if has_vocab else []

    def pick(lg):
        if sampler is None:
            return greedy_argmax(lg)
        return int(sampler(lg, prompt_ids + ids, len(ids)))

    if has_vocab:
        lg = lm_head_logits(out[-1], glob["final_norm"], table, cfg.eps, prec)
        res["logits0"] = lg
        ids.append(pick(lg))
        margins.append(_top2_margin(lg))
    res["t_prefill_s"] = time.perf_counter() - t_start
    t_start = time.perf_counter()
    for i in range(steps):
        pos = S + i
        if pos >= W:
            raise ValueError("decode position exceeds the KV window")
        if has_vocab:
            feed = ids[-1] if forced_ids is None else int(forced_ids[i])
            row = table[feed][None, :].astype(np.float64)
        else:
            row = np.asarray(glob["decode_x"][i], np.float64)[None, :]
        hx = stack(row, pos)
        dec_x.append(hx[0])
        if has_vocab:
            lg = lm_head_logits(hx[0], glob["final_norm"], table, cfg.eps, prec)
            ids.append(pick(lg))
            margins.append(_top2_margin(lg))
            if keep_logits:
                all_logits.append(lg)
    res["t_decode_s"] = time.perf_counter() - t_start
    res["ids"] = np.asarray(ids, np.int64)
    res["margins"] = np.asarray(margins)
    res["decode_x"] = np.asarray(dec_x).reshape(steps, cfg.hidden)
    if keep_logits:
        res["step_logits"] = all_logits
    return res


def block_logits(cfg, glob, layers, block_ids, prec=None):
    """Logits of every row of a token block appended to the prompt, by definition:
    one causal forward over prompt + block (embedding, image injection, every
    layer over the whole sequence), final RMSNorm and lm_head on each block row.

    This is what a multi-token verify of a drafted block computes ([HyOCR15]
    §3.8: the target checks the drafted tokens in one causal forward): row i's
    logits pick the token that follows prompt + block[0..i].
    Returns [len(block_ids), V] float64.
    """
    if prec is None:
        prec = BF16 if cfg.dtype == "bf16" else F64
    block_ids = [int(i) for i in block_ids]
    S, k = len(glob["ids"]), len(block_ids)
    W = S + k
    ws = [_prep_weights(w, prec) for w in layers]
    table = np.asarray(glob["embed"], np.float32 if prec == BF16_F32SUM else np.float64)
    x = embed_inject(glob["embed"], glob["ids"], cfg.placeholder_id, glob.get("img"))
    x = np.concatenate([x, table[block_ids].astype(np.float64)], axis=0)
    cos, sin = rope_tables(np.arange(W)[None, :], np.zeros(cfg.head_dim // 2, np.int64), 1, cfg.head_dim, cfg.theta)
    for l in range(cfg.n_layers):
        kc = np.zeros((cfg.n_kv_heads, W, cfg.head_dim))
        vc = np.zeros_like(kc)
        x = decoder_layer(x, ws[l], cfg, kc, vc, 0, cos, sin, prec)
    return np.stack([lm_head_logits(x[S + i], glob["final_norm"], table, cfg.eps, prec) for i in range(k)])
