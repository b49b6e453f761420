"""Naive pure-Python loop implementations for tiny shapes.

Written independently of oracle/ (no imports from it, scalar loops only) so
that the vectorised oracle can be checked against them. Every formula below is
restated from the pages: RMSNorm / LayerNorm, the textbook rotation form of
RoPE (complex multiplication), written-out softmax, GQA head mapping through
repeat_interleave expansion, SwiGLU, pre-LN ViT block.

bf16 forms: `bf16` rounds a Python float to the nearest bfloat16 from its
IEEE-754 double bits (8 significant bits, ties to even); the layer functions
take an optional rounding op applied at the points where the bf16 policy
stores a value (operands of every projection, q and the cached k/v), and
their dot products then use math.fsum (correctly rounded sums).
"""
import math
import struct


def bf16(v):
    """Nearest bfloat16 value of a finite double (round half to even), as a float.

    A double holds 52 explicit mantissa bits, a bfloat16 7: the low 45 bits are
    dropped, rounding the kept part up when they exceed half an ulp, or equal
    it with an odd kept part (a carry into the exponent is the correct result).
    Values in the bf16 normal range only (the workloads produce no others)."""
    if v == 0.0:
        return v
    b = struct.unpack("<Q", struct.pack("<d", v))[0]
    drop = 45
    low = b & ((1 << drop) - 1)
    b >>= drop
    half = 1 << (drop - 1)
    if low > half or (low == half and (b & 1)):
        b += 1
    return struct.unpack("<d", struct.pack("<Q", b << drop))[0]


def matvec_exact(W, x):
    """W [n][k] times x [k] with correctly rounded sums (math.fsum)."""
    return [math.fsum(W[i][j] * x[j] for j in range(len(x))) for i in range(len(W))]


def matvec(W, x):
    """W [n][k] times x [k]."""
    return [sum(W[i][j] * x[j] for j in range(len(x))) for i in range(len(W))]


def rmsnorm(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def layernorm(x, g, b, eps):
    n = len(x)
    mu = sum(x) / n
    var = sum((v - mu) ** 2 for v in x) / n
    r = 1.0 / math.sqrt(var + eps)
    return [(x[i] - mu) * r * g[i] + b[i] for i in range(n)]


def rope_complex(u, angles):
    """Rotate consecutive-half pairs (u[j], u[j+h]) as the complex number
    u[j] + i u[j+h] multiplied by exp(i angle_j)."""
    h = len(u) // 2
    out = [0.0] * len(u)
    for j in range(h):
        a, b = u[j], u[j + h]
        c, s = math.cos(angles[j]), math.sin(angles[j])
        out[j] = a * c - b * s
        out[j + h] = a * s + b * c
    return out


def rope_complex_adjacent(u, angles):
    """Rotate adjacent pairs (u[2j], u[2j+1]) as the complex number
    u[2j] + i u[2j+1] multiplied by exp(i angle_j); the real part goes to
    element j, the imaginary part to element j + d/2."""
    h = len(u) // 2
    out = [0.0] * len(u)
    for j in range(h):
        z = complex(u[2 * j], u[2 * j + 1]) * complex(math.cos(angles[j]), math.sin(angles[j]))
        out[j] = z.real
        out[j + h] = z.imag
    return out


def text_angles(pos, d, theta):
    return [pos * theta ** (-2.0 * j / d) for j in range(d // 2)]


def silu(z):
    return z / (1.0 + math.exp(-z))


def gelu_tanh(z):
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def attention_rows(qs, ks, vs, visible):
    """qs [Sq][d]; ks, vs [Sk][d]; visible(i, j) -> bool. Softmax written out."""
    d = len(qs[0])
    out = []
    for i, q in enumerate(qs):
        scores = []
        for j, k in enumerate(ks):
            if visible(i, j):
                scores.append((j, sum(q[t] * k[t] for t in range(d)) / math.sqrt(d)))
        m = max(s for _, s in scores)
        e = [(j, math.exp(s - m)) for j, s in scores]
        tot = sum(v for _, v in e)
        o = [0.0] * len(vs[0])
        for j, p in e:
            for t in range(len(o)):
                o[t] += p / tot * vs[j][t]
        out.append(o)
    return out


def expand_kv_rows(W, n_kv, head_dim, rep):
    """Repeat each KV head's block of rows `rep` times consecutively
    (repeat_interleave over heads), as the GQA-to-MHA weight expansion does."""
    out = []
    for g in range(n_kv):
        block = W[g * head_dim:(g + 1) * head_dim]
        for _ in range(rep):
            out.extend([list(r) for r in block])
    return out


def decoder_layer_mha(xs, w, nq, d, eps, theta, qk_norm, pos0, cache_k, cache_v, interleave=False, rnd=None):
    """One decoder layer written as MHA over expanded K/V weights.

    xs: list of rows at positions pos0..; w: dict of nested lists with wk/wv
    already expanded to nq heads; cache_k/cache_v: lists (per position) of
    [nq][d] rows, extended in place. qk_norm: 0 none, 1 (or True) per-head
    RMSNorm before the rotation, 2 after it. interleave: rotate adjacent pairs.
    rnd: None (plain float64), or f(vec, tag) -> vec, the storage rounding
    applied at each point tagged "h" (normed row), "q", "k", "v" (after the
    rotation), "o" (attention output), "h2" (post-attention normed row) and
    "a" (SwiGLU product); projections then use correctly rounded sums.
    """
    rot = rope_complex_adjacent if interleave else rope_complex
    mv = matvec if rnd is None else matvec_exact
    r = (lambda vec, tag: vec) if rnd is None else rnd
    outs = []
    for s, x in enumerate(xs):
        pos = pos0 + s
        h = r(rmsnorm(x, w["attn_norm"], eps), "h")
        q = mv(w["wq"], h)
        k = mv(w["wk"], h)
        v = mv(w["wv"], h)
        qh, kh, vh = [], [], []
        for hd in range(nq):
            qq = q[hd * d:(hd + 1) * d]
            kk = k[hd * d:(hd + 1) * d]
            if int(qk_norm) == 1:
                qq = rmsnorm(qq, w["q_norm"], eps)
                kk = rmsnorm(kk, w["k_norm"], eps)
            ang = text_angles(pos, d, theta)
            qq, kk = rot(qq, ang), rot(kk, ang)
            if int(qk_norm) == 2:
                qq = rmsnorm(qq, w["q_norm"], eps)
                kk = rmsnorm(kk, w["k_norm"], eps)
            qh.append(r(qq, "q"))
            kh.append(r(kk, "k"))
            vh.append(r(v[hd * d:(hd + 1) * d], "v"))
        cache_k.append(kh)
        cache_v.append(vh)
        o = []
        for hd in range(nq):
            ks = [cache_k[j][hd] for j in range(pos + 1)]
            vs = [cache_v[j][hd] for j in range(pos + 1)]
            o.extend(attention_rows([qh[hd]], ks, vs, lambda i, j: True)[0])
        att = mv(w["wo"], r(o, "o"))
        x = [x[i] + att[i] for i in range(len(x))]
        h2 = r(rmsnorm(x, w["mlp_norm"], eps), "h2")
        g = mv(w["wg"], h2)
        u = mv(w["wu"], h2)
        a = r([silu(g[i]) * u[i] for i in range(len(g))], "a")
        dn = mv(w["wd"], a)
        outs.append([x[i] + dn[i] for i in range(len(x))])
    return outs


def vit_layer(xs, w, nh, d, eps, pos_hw, theta, visible, rnd=None):
    """Pre-LN ViT block; 2D RoPE: first half of each head by h, second by w.
    rnd: as in decoder_layer_mha, with tags "h", "q", "k", "v", "o", "h2" and
    "f" (GELU output); correctly rounded projection sums."""
    mv = matvec if rnd is None else matvec_exact
    r = (lambda vec, tag: vec) if rnd is None else rnd
    S = len(xs)
    q_all, k_all, v_all = [], [], []
    for s in range(S):
        h = r(layernorm(xs[s], w["attn_norm"], w["attn_norm_b"], eps), "h")
        q = [a + b for a, b in zip(mv(w["wq"], h), w["bq"])]
        k = [a + b for a, b in zip(mv(w["wk"], h), w["bk"])]
        v = [a + b for a, b in zip(mv(w["wv"], h), w["bv"])]
        qr, kr = [], []
        for hd in range(nh):
            qq, kk = q[hd * d:(hd + 1) * d], k[hd * d:(hd + 1) * d]
            half = d // 2
            ah = text_angles(pos_hw[0][s], half, theta)
            aw = text_angles(pos_hw[1][s], half, theta)
            qr.append(r(rope_complex(qq[:half], ah) + rope_complex(qq[half:], aw), "q"))
            kr.append(r(rope_complex(kk[:half], ah) + rope_complex(kk[half:], aw), "k"))
        q_all.append(qr)
        k_all.append(kr)
        v_all.append([r(v[hd * d:(hd + 1) * d], "v") for hd in range(nh)])
    outs = []
    for s in range(S):
        o = []
        for hd in range(nh):
            o.extend(attention_rows([q_all[s][hd]], [k_all[j][hd] for j in range(S)],
                                    [v_all[j][hd] for j in range(S)], lambda i, j: visible(s, j))[0])
        att = [a + b for a, b in zip(mv(w["wo"], r(o, "o")), w["bo"])]
        x = [xs[s][i] + att[i] for i in range(len(att))]
        h2 = r(layernorm(x, w["mlp_norm"], w["mlp_norm_b"], eps), "h2")
        f = r([gelu_tanh(a + b) for a, b in zip(mv(w["w1"], h2), w["b1"])], "f")
        dn = [a + b for a, b in zip(mv(w["w2"], f), w["b2"])]
        outs.append([x[i] + dn[i] for i in range(len(x))])
    return outs
