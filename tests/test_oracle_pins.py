"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test targets a mistake that could hide in the oracle (dropped gain, wrong
rotate-half sign, wrong GQA head mapping, mask leak, wrong permutation, ...).
All CPU; shapes are tiny except where a page's own count is checked.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import decoder as od
from oracle import vit as ov
import vlm_synth as vs
from tests import _brute as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def pages():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- bf16
def test_bf16_round_matches_library_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10 ** rng.uniform(-3, 3, 20000).astype(np.float32),
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 65504.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(od.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_and_overflow():
    assert od.bf16_round(1.0 + 2 ** -8) == 1.0               # tie -> even (down)
    assert od.bf16_round(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6  # tie -> even (up)
    assert od.bf16_round(1.0 + 2 ** -8 + 2 ** -20) == 1.0 + 2 ** -7
    assert np.isinf(od.bf16_round(3.5e38))
    assert od.bf16_round(3.0e38) == pytest.approx(3.0e38, rel=2 ** -8)


def test_synth_bf16_values_agree_with_oracle_rounding():
    x = np.random.default_rng(1).standard_normal(5000).astype(np.float32)
    assert np.array_equal(vs.to_bf16_values(x).astype(np.float64), od.bf16_round(x.astype(np.float64)))


# ----------------------------------------------------------------------------- norms
def test_rms_norm_closed_form_constant_row():
    c, eps = 0.37, 1e-6
    g = np.linspace(0.5, 1.5, 16)
    y = od.rms_norm(np.full(16, c), g, eps)
    assert np.allclose(y, g * c / math.sqrt(c * c + eps), rtol=1e-15)


def test_rms_norm_unit_rms_and_scale_invariance():
    x = np.random.default_rng(2).standard_normal((4, 64))
    y = od.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)
    assert np.allclose(od.rms_norm(7.5 * x, np.ones(64), 1e-12), od.rms_norm(x, np.ones(64), 1e-12), rtol=1e-10)


def test_rms_norm_matches_brute_force():
    rng = np.random.default_rng(3)
    x, g = rng.standard_normal(12), rng.standard_normal(12)
    assert np.allclose(od.rms_norm(x, g, 1e-6), bf.rmsnorm(list(x), list(g), 1e-6), rtol=1e-13)


def test_layer_norm_moments_and_brute_force():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 40)) * 3 + 2
    y = od.layer_norm(x, np.ones(40), np.zeros(40), 0.0)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-14)
    assert np.allclose((y * y).mean(axis=1), 1, rtol=1e-13)
    g, b = rng.standard_normal(40), rng.standard_normal(40)
    assert np.allclose(od.layer_norm(x[0], g, b, 1e-6), bf.layernorm(list(x[0]), list(g), list(b), 1e-6), rtol=1e-12)


# ----------------------------------------------------------------------------- activations
def test_silu_identities():
    z = np.linspace(-20, 20, 401)
    assert od.silu(0.0) == 0.0
    assert np.allclose(od.silu(z) - od.silu(-z), z, atol=1e-12)      # z*s(z) - (-z)*s(-z) = z
    assert od.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert np.allclose(od.silu(z[:5]), [bf.silu(v) for v in z[:5]], rtol=1e-14)


def test_gelu_tanh_against_erf_form():
    from scipy.special import erf
    z = np.linspace(-6, 6, 241)
    exact = 0.5 * z * (1 + erf(z / math.sqrt(2)))
    assert np.max(np.abs(od.gelu_tanh(z) - exact)) < 1e-3          # tanh approximation error
    assert np.allclose(od.gelu_tanh(z) - od.gelu_tanh(-z), z, atol=1e-12)
    assert od.gelu_tanh(0.0) == 0.0


# ----------------------------------------------------------------------------- RoPE
def _text_tables(T, d, theta=1e6):
    return od.rope_tables(np.arange(T)[None, :], np.zeros(d // 2, np.int64), 1, d, theta)


def test_rope_position_zero_is_identity():
    cos, sin = _text_tables(4, 64)
    u = np.random.default_rng(5).standard_normal((1, 3, 64))
    assert np.array_equal(od.rope_apply(u, cos[:1], sin[:1], 1), u)


def test_rope_matches_complex_rotation():
    d, T = 16, 9
    cos, sin = _text_tables(T, d, 1e4)
    u = np.random.default_rng(6).standard_normal((T, 2, d))
    y = od.rope_apply(u, cos, sin, 1)
    for t in range(T):
        for h in range(2):
            assert np.allclose(y[t, h], bf.rope_complex(list(u[t, h]), bf.text_angles(t, d, 1e4)), rtol=1e-13, atol=1e-14)


def test_rope_pm1_matrix_form():
    """Youtu-VL ncnn port, 实现难点 §2: rotate-half as a constant +-1 matrix, (q@P)cos + (q@PR)sin with P = I."""
    d = 64
    R = np.zeros((d, d))
    for j in range(d // 2):
        R[j + d // 2, j] = -1.0
        R[j, j + d // 2] = 1.0
    cos, sin = _text_tables(11, d)
    q = np.random.default_rng(7).standard_normal((11, 1, d))
    ref = q[:, 0] * cos + (q[:, 0] @ R) * sin
    assert np.allclose(od.rope_apply(q, cos, sin, 1)[:, 0], ref, rtol=1e-14, atol=1e-15)


def test_rope_norm_preserving_and_relative():
    d = 128
    cos, sin = _text_tables(200, d)
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    rq = lambda m, v: od.rope_apply(v[None, None, :], cos[m:m + 1], sin[m:m + 1], 1)[0, 0]
    assert np.linalg.norm(rq(57, q)) == pytest.approx(np.linalg.norm(q), rel=1e-13)
    for m, n in [(5, 3), (150, 20), (199, 199)]:
        assert rq(m, q) @ rq(n, k) == pytest.approx(rq(m - n, q) @ k, rel=1e-10, abs=1e-10)


def test_rope_table_values_closed_form():
    cos, sin = _text_tables(50, 128, 1e6)
    t = np.arange(50)
    assert np.allclose(cos[:, 0], np.cos(t)) and np.allclose(cos[:, 64], np.cos(t))
    assert np.allclose(sin[:, 63], np.sin(t * 1e6 ** (-126 / 128)))


def test_rope_two_segments_equal_two_1d_ropes():
    d, T = 72, 13
    rng = np.random.default_rng(9)
    pos = rng.integers(0, 40, size=(2, T))
    axes = np.r_[np.zeros(18, np.int64), np.ones(18, np.int64)]
    cos, sin = od.rope_tables(pos, axes, 2, d, 1e6)
    u = rng.standard_normal((T, 3, d))
    y = od.rope_apply(u, cos, sin, 2)
    c0, s0 = od.rope_tables(pos[:1], np.zeros(18, np.int64), 1, 36, 1e6)
    c1, s1 = od.rope_tables(pos[1:], np.zeros(18, np.int64), 1, 36, 1e6)
    assert np.allclose(y[..., :36], od.rope_apply(u[..., :36], c0, s0, 1), rtol=1e-14)
    assert np.allclose(y[..., 36:], od.rope_apply(u[..., 36:], c1, s1, 1), rtol=1e-14)


def test_rope_multi_axis_equal_axes_is_text_rope():
    d, T = 64, 20
    pos = np.tile(np.arange(T), (4, 1))
    axes = np.repeat(np.arange(4), 8)                  # sections [8,8,8,8] over 32 pairs
    c, s = od.rope_tables(pos, axes, 1, d, 1e6)
    c1, s1 = _text_tables(T, d)
    assert np.array_equal(c, c1) and np.array_equal(s, s1)


def test_interleaved_rope_matches_adjacent_pair_rotation():
    """Youtu-VL ncnn port, 实现难点 §2: pairs of adjacent elements turn together
    and land in the two halves of the head."""
    d, T = 16, 9
    cos, sin = _text_tables(T, d, 1e4)
    u = np.random.default_rng(61).standard_normal((T, 2, d))
    y = od.rope_apply(u, cos, sin, 1, interleave=True)
    for t in range(T):
        for h in range(2):
            ref = bf.rope_complex_adjacent(list(u[t, h]), bf.text_angles(t, d, 1e4))
            assert np.allclose(y[t, h], ref, rtol=1e-13, atol=1e-14)


def test_interleaved_rope_is_a_permutation_then_rotation():
    """The de-interleave is the fixed permutation P of the page (q @ P): a
    permutation matrix, position 0 gives q @ P, and q.k is invariant under it."""
    d = 64
    P = np.zeros((d, d))
    for j in range(d // 2):
        P[2 * j, j] = 1.0
        P[2 * j + 1, j + d // 2] = 1.0
    cos, sin = _text_tables(40, d)
    rng = np.random.default_rng(62)
    q, k = rng.standard_normal((2, 1, 1, d))
    assert np.array_equal(od.rope_apply(q, cos[:1], sin[:1], 1, interleave=True)[0, 0], q[0, 0] @ P)
    rq = lambda m, v: od.rope_apply(v, cos[m:m + 1], sin[m:m + 1], 1, interleave=True)[0, 0]
    for m, n in [(7, 3), (39, 0)]:
        assert rq(m, q) @ rq(n, k) == pytest.approx(rq(m - n, q) @ (k[0, 0] @ P), rel=1e-10, abs=1e-10)


def test_alpha_scaled_base_matches_page():
    """HunyuanOCR v1.0 ncnn port, 二 and 五.1: base = theta * alpha^(d/(d-2)),
    printed as ~1.11588e7 for its 128-wide heads (four 16-pair sections)."""
    p = pages()["hunyuan_xdrope_base"]
    d = p["head_dim"]
    assert 4 * 16 * 2 == d
    assert od.alpha_scaled_base(1e6, 1.0, d) == 1e6            # alpha 1: the plain base
    b = od.alpha_scaled_base(p["rope_theta"], p["alpha"], d)
    assert b == pytest.approx(p["value"], rel=5e-6)
    assert math.log(b / p["rope_theta"]) == pytest.approx(math.log(p["alpha"]) * d / (d - 2), rel=1e-12)
    # the page: frequencies of pairs j >= 32 (the last two axes) are near zero
    inv = b ** (-2.0 * np.arange(d // 2) / d)
    assert inv[32] < 3.1e-4 and inv[63] < 1.3e-7 and inv[0] == 1.0


def test_qk_norm_orders():
    """HunyuanOCR v1.0 ncnn port, 五.2: norm after the rotation, and the cache
    holds the normalised k; with a unit gain both orders agree (a rotation
    keeps each head's RMS), with a general gain they do not."""
    cfg2 = vs.scaled(TINY, qk_norm=2, eps=0.0)   # eps 0: the normalised rows have RMS exactly 1
    cfg1 = vs.scaled(TINY, qk_norm=1, eps=0.0)
    w = {k: v.astype(np.float64) for k, v in vs.decoder_layer_weights(cfg2, 0).items()}
    x = np.random.default_rng(63).standard_normal((cfg2.seq, cfg2.hidden))
    cos, sin = _text_tables(cfg2.capacity, cfg2.head_dim, cfg2.theta)

    def run(cfg, ww):
        kc = np.zeros((cfg.n_kv_heads, cfg.capacity, cfg.head_dim)); vc = np.zeros_like(kc)
        return od.decoder_layer(x, ww, cfg, kc, vc, 0, cos, sin, od.F64), kc

    y2, k2 = run(cfg2, w)
    y1, k1 = run(cfg1, w)
    assert not np.allclose(y1, y2, rtol=1e-6)
    ms = np.mean((k2[:, :cfg2.seq] / w["k_norm"]) ** 2, axis=-1)   # normalised after the rotation
    assert np.allclose(ms, 1.0, rtol=0, atol=1e-12)
    ms1 = np.mean((k1[:, :cfg1.seq] / w["k_norm"]) ** 2, axis=-1)
    assert not np.allclose(ms1, 1.0, atol=1e-2)
    u = dict(w, q_norm=np.ones(cfg2.head_dim), k_norm=np.ones(cfg2.head_dim))
    assert np.allclose(run(cfg2, u)[0], run(cfg1, u)[0], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- expanded MLA
MLA_TINY = vs.scaled(vs.C_MLA, hidden=64, n_q_heads=3, n_kv_heads=3, head_dim=24, qk_rope_dim=8, v_head_dim=16,
                     q_lora_rank=32, kv_lora_rank=40, ffn=96, vocab=0, seq=7, n_img=0, img_start=0, capacity=8)


def test_mla_expanded_equals_absorbed_latent_form():
    """Youtu-VL-4B ncnn port, 实现流程 §6: the port expands the latent with kv_b instead of absorbing
    it. Absorbing (q_nope . W_uk c = (W_uk^T q_nope) . c, o = W_uv sum_j p_j c_j) is the same
    function; computing it that way pins the per-head split of kv_b, the shared rotated key, the
    head layout of the cache and the 1/sqrt(dn + dr) scale."""
    cfg = MLA_TINY
    w = {k: v.astype(np.float64) for k, v in vs.decoder_layer_weights(cfg, 0).items()}
    rng = np.random.default_rng(71)
    S, nq, d, dr, dv, r = cfg.seq, cfg.n_q_heads, cfg.head_dim, cfg.qk_rope_dim, cfg.v_head_dim, cfg.kv_lora_rank
    dn = d - dr
    x = rng.standard_normal((S, cfg.hidden))
    cos, sin = _text_tables(cfg.capacity, dr, cfg.theta)
    kc = np.zeros((nq, cfg.capacity, d)); vc = np.zeros((nq, cfg.capacity, dv))
    got = od.mla_layer(x, w, cfg, kc, vc, 0, cos, sin, od.F64)
    # absorbed form, written per head and per key
    h = od.rms_norm(x, w["attn_norm"], cfg.eps)
    q = od.rms_norm(h @ w["wq_a"].T, w["q_a_norm"], cfg.eps) @ w["wq_b"].T
    ckv = h @ w["wkv_a"].T
    c = od.rms_norm(ckv[:, :r], w["kv_a_norm"], cfg.eps)
    att = np.zeros((S, nq * dv))
    for i in range(nq):
        wb = w["wkv_b"][i * (dn + dv):(i + 1) * (dn + dv)]
        w_uk, w_uv = wb[:dn], wb[dn:]
        for t in range(S):
            qn = q[t, i * d:i * d + dn]
            qr = od.rope_apply(q[t, None, None, i * d + dn:(i + 1) * d], cos[t:t + 1], sin[t:t + 1], 1, True)[0, 0]
            sc = []
            for j in range(t + 1):
                kr = od.rope_apply(ckv[j, None, None, r:], cos[j:j + 1], sin[j:j + 1], 1, True)[0, 0]
                sc.append(((w_uk.T @ qn) @ c[j] + qr @ kr) / math.sqrt(d))
            sc = np.array(sc)
            p = np.exp(sc - sc.max()); p /= p.sum()
            att[t, i * dv:(i + 1) * dv] = w_uv @ (p @ c[:t + 1])
    y = x + att @ w["wo"].T
    h2 = od.rms_norm(y, w["mlp_norm"], cfg.eps)
    g = h2 @ w["wg"].T
    ref = y + ((g / (1 + np.exp(-g))) * (h2 @ w["wu"].T)) @ w["wd"].T
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)
    # the cache holds the expanded per-head keys (192-style width) and values (128-style width)
    assert kc.shape[-1] == dn + dr and vc.shape[-1] == dv
    assert np.allclose(vc[0, :S], c @ w["wkv_b"][dn:dn + dv].T, rtol=1e-12)
    assert np.allclose(kc[1, :S, :dn], c @ w["wkv_b"][(dn + dv):(dn + dv) + dn].T, rtol=1e-12)
    kr = od.rope_apply(ckv[:, None, r:], cos[:S], sin[:S], 1, True)[:, 0]   # [nope | rope], rope shared
    for i in range(nq):
        assert np.allclose(kc[i, :S, dn:], kr, rtol=1e-12, atol=1e-14)


def test_mla_cache_shapes_match_page():
    """Youtu-VL-4B ncnn port, 实现流程 §6-§7: per-layer K [32, 512, 192], V [32, 512, 128], nkv = nq."""
    p = pages()["youtu_kv_window"]
    cfg = vs.scaled(vs.C_MLA, n_q_heads=32, n_kv_heads=32, capacity=p["window"])
    assert [cfg.n_kv_heads, cfg.capacity, cfg.head_dim] == p["k_shape"]
    assert [cfg.n_kv_heads, cfg.capacity, cfg.v_head_dim] == p["v_shape"]
    assert cfg.head_dim - cfg.qk_rope_dim == 128 and cfg.kv_lora_rank == 512 and cfg.qk_rope_dim == 64


def test_mla_prefill_equals_decode_replay():
    cfg = vs.scaled(MLA_TINY, n_layers=2, seq=7, capacity=8)
    glob = {"x": np.random.default_rng(72).standard_normal((cfg.seq, cfg.hidden))}
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(2)]
    a = od.run_decoder(cfg, glob, layers, steps=0)
    b = od.run_decoder(cfg, glob, layers, steps=0, prefill_split=3)
    assert np.allclose(a["prefill_x"], b["prefill_x"], rtol=1e-12, atol=1e-12)
    assert np.allclose(a["k_cache"], b["k_cache"], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- sampling
from oracle import sampling as osm


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def test_sampling_repetition_penalty_worked_example():
    """HunyuanOCR v1.5 port §3.6/§4 name the penalty; reading: x/r for x > 0, x*r otherwise, once per id."""
    got = osm.penalize([2.0, -1.0, 0.5, 3.0], [0, 1, 1], 2.0)
    assert np.array_equal(got, [1.0, -2.0, 0.5, 3.0])


def test_sampling_top_k_one_and_tiny_top_p_are_argmax():
    c = vs.sampling_case(1, 500, 20, n_draws=50)
    pen = osm.penalize(c["logits"], c["context"], 1.3)
    best = int(np.argmax(pen))
    for u in c["u"]:
        assert osm.sample_token(c["logits"], c["context"], 0.7, 1, 1.0, 1.3, float(u))[0] == best
        assert osm.sample_token(c["logits"], c["context"], 0.7, 0, 1e-9, 1.3, float(u))[0] == best


def test_sampling_draws_follow_softmax_over_the_kept_set():
    """Over an evenly spaced grid of u the draw counts are N p within 1 (inverse CDF), where p is
    the softmax of the tempered, penalised logits over the top-k set, computed here on its own."""
    c = vs.sampling_case(2, 60, 10)
    N, T, k = 4000, 1.7, 25
    x = osm.penalize(c["logits"], c["context"], 1.5) / T
    top = np.argsort(-x, kind="stable")[:k]
    p = np.zeros(60)
    p[top] = _softmax(x[top])
    counts = np.zeros(60)
    for i in range(N):
        counts[osm.sample_token(c["logits"], c["context"], T, k, 1.0, 1.5, (i + 0.5) / N)[0]] += 1
    assert np.all(np.abs(counts - N * p) <= 1.0 + 1e-9)
    assert counts[np.setdiff1d(np.arange(60), top)].sum() == 0


def test_sampling_top_p_keeps_the_crossing_token():
    """[MNN] §4.1: sorted by probability, tokens after the cumulative passes the threshold are cut."""
    x = np.log([0.5, 0.3, 0.2])
    kept = lambda p: osm.sample_token(x, [], 1.0, 0, p, 1.0, 0.0)[1]["kept"]
    assert kept(0.6) == 2 and kept(0.49) == 1 and kept(0.81) == 3 and kept(0.79) == 2
    # u just below the first token's share of the kept mass picks it, just above picks the next
    assert osm.sample_token(x, [], 1.0, 0, 0.6, 1.0, 0.62)[0] == 0
    assert osm.sample_token(x, [], 1.0, 0, 0.6, 1.0, 0.63)[0] == 1


def test_sampling_temperature_scales_logits():
    c = vs.sampling_case(3, 40, 0)
    N, T = 3000, 2.5
    p = _softmax(c["logits"].astype(np.float64) / T)
    counts = np.bincount([osm.sample_token(c["logits"], [], T, 0, 1.0, 1.0, (i + 0.5) / N)[0] for i in range(N)],
                         minlength=40)
    assert np.all(np.abs(counts - N * p) <= 1.0 + 1e-9)


# ----------------------------------------------------------------------------- attention
def test_attention_matches_brute_force_with_mask():
    rng = np.random.default_rng(10)
    q, k, v = rng.standard_normal((1, 5, 8)), rng.standard_normal((1, 7, 8)), rng.standard_normal((1, 7, 6))
    vis = rng.random((5, 7)) < 0.6
    vis[:, 0] = True
    mask = np.where(vis, 0.0, od.MASK_NEG)
    got = od.softmax_attention(q, k, v, mask, 1)[0]
    ref = bf.attention_rows(q[0].tolist(), k[0].tolist(), v[0].tolist(), lambda i, j: bool(vis[i, j]))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_attention_single_key_and_zero_query():
    rng = np.random.default_rng(11)
    k, v = rng.standard_normal((1, 6, 4)), rng.standard_normal((1, 6, 4))
    q = rng.standard_normal((1, 6, 4))
    o = od.softmax_attention(q, k, v, od.window_mask(6, 0, 6), 1)[0]
    assert np.allclose(o[0], v[0, 0], rtol=1e-15)                      # only key 0 visible
    o0 = od.softmax_attention(np.zeros((1, 6, 4)), k, v, od.window_mask(6, 0, 6), 1)[0]
    for i in range(6):
        assert np.allclose(o0[i], v[0, :i + 1].mean(axis=0), rtol=1e-13)


def test_gqa_equals_mha_with_repeat_interleaved_kv():
    rng = np.random.default_rng(12)
    nq, nkv = 8, 2
    q, k, v = rng.standard_normal((nq, 5, 4)), rng.standard_normal((nkv, 5, 4)), rng.standard_normal((nkv, 5, 4))
    m = od.window_mask(5, 0, 5)
    gqa = od.softmax_attention(q, k, v, m, nq // nkv)
    mha = od.softmax_attention(q, np.repeat(k, nq // nkv, axis=0), np.repeat(v, nq // nkv, axis=0), m, 1)
    assert np.array_equal(gqa, mha)


def test_window_mask_equals_truncation():
    rng = np.random.default_rng(13)
    W, S, pos0 = 16, 3, 5
    q = rng.standard_normal((2, S, 8))
    k = rng.standard_normal((1, W, 8)) * 50      # garbage in unfilled slots must not leak
    v = rng.standard_normal((1, W, 8)) * 50
    full = od.softmax_attention(q, k, v, od.window_mask(S, pos0, W), 2)
    for s in range(S):
        T = pos0 + s + 1
        trunc = od.softmax_attention(q[:, s:s + 1], k[:, :T], v[:, :T], np.zeros((1, T)), 2)
        # masked slots get weight exp(-1e9 - m) == 0 exactly; only BLAS summation order differs
        assert np.allclose(full[:, s:s + 1], trunc, rtol=1e-13, atol=1e-13)


def test_mask_constants_match_pages():
    p = pages()["youtu_kv_window"]
    assert od.MASK_NEG == p["mask_invalid"]
    m = od.window_mask(2, 3, 6)
    assert list(m[0]) == [0, 0, 0, 0, p["mask_invalid"], p["mask_invalid"]]


# ----------------------------------------------------------------------------- embed / head
def test_embed_inject_rows_and_count_check():
    E = np.arange(40, dtype=np.float64).reshape(10, 4)
    ids = np.array([1, 9, 9, 3, 9, 2])
    img = -np.arange(12, dtype=np.float64).reshape(3, 4) - 1
    x = od.embed_inject(E, ids, 9, img)
    assert np.array_equal(x[[0, 3, 5]], E[[1, 3, 2]])
    assert np.array_equal(x[[1, 2, 4]], img)
    with pytest.raises(ValueError):
        od.embed_inject(E, ids, 9, img[:2])


def test_greedy_argmax_ties_nan_signed_zero():
    assert od.greedy_argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert od.greedy_argmax([-0.0, 0.0, -1.0]) == 0
    assert od.greedy_argmax([-2.0, -0.0, 0.0]) == 1
    with pytest.raises(FloatingPointError):
        od.greedy_argmax([1.0, np.nan])
    with pytest.raises(FloatingPointError):
        od.greedy_argmax([1.0, np.inf])


def test_lm_head_matches_brute_force():
    rng = np.random.default_rng(14)
    E, x, g = rng.standard_normal((9, 6)), rng.standard_normal(6), rng.standard_normal(6)
    lg = od.lm_head_logits(x, g, E, 1e-6, od.F64)
    assert np.allclose(lg, bf.matvec(E.tolist(), bf.rmsnorm(list(x), list(g), 1e-6)), rtol=1e-13)


# ----------------------------------------------------------------------------- decoder layer
TINY = vs.DecoderConfig("tiny", 99, n_layers=2, hidden=8, n_q_heads=4, n_kv_heads=2, head_dim=4, ffn=6,
                        vocab=16, seq=5, n_img=2, img_start=1, decode_steps=3, capacity=8, dtype="f32",
                        qk_norm=True, theta=1e4)


@pytest.mark.parametrize("qk_norm,interleave", [(1, False), (0, False), (2, False), (0, True), (2, True)])
def test_decoder_layer_matches_brute_force_mha(qk_norm, interleave):
    cfg = vs.scaled(TINY, qk_norm=qk_norm, rope_interleave=interleave)
    w = {k: v.astype(np.float64) for k, v in vs.decoder_layer_weights(cfg, 0).items()}
    x = np.random.default_rng(15).standard_normal((cfg.seq, cfg.hidden))
    cos, sin = _text_tables(cfg.capacity, cfg.head_dim, cfg.theta)
    kc = np.zeros((cfg.n_kv_heads, cfg.capacity, cfg.head_dim)); vc = np.zeros_like(kc)
    got = od.decoder_layer(x, w, cfg, kc, vc, 0, cos, sin, od.F64)
    rep = cfg.n_q_heads // cfg.n_kv_heads
    wl = {k: v.tolist() for k, v in w.items()}
    wl["wk"] = bf.expand_kv_rows(wl["wk"], cfg.n_kv_heads, cfg.head_dim, rep)
    wl["wv"] = bf.expand_kv_rows(wl["wv"], cfg.n_kv_heads, cfg.head_dim, rep)
    ck, cv = [], []
    ref = bf.decoder_layer_mha(x.tolist(), wl, cfg.n_q_heads, cfg.head_dim, cfg.eps, cfg.theta, qk_norm, 0, ck, cv,
                               interleave)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)
    # the cache holds the roped, normed K of each KV head
    for s in range(cfg.seq):
        for g in range(cfg.n_kv_heads):
            assert np.allclose(kc[g, s], ck[s][g * rep], rtol=1e-12, atol=1e-14)
            assert np.allclose(vc[g, s], cv[s][g * rep], rtol=1e-12, atol=1e-14)


def test_gqa_layer_equals_penguin_weight_expansion():
    """Penguin-VL ncnn port §3: expanding the K/V weights per head with
    repeat_interleave turns the GQA layer into an MHA layer with the same output."""
    cfg = vs.scaled(TINY, qk_norm=True)
    w = {k: v.astype(np.float64) for k, v in vs.decoder_layer_weights(cfg, 1).items()}
    rep = cfg.n_q_heads // cfg.n_kv_heads
    H, d = cfg.hidden, cfg.head_dim
    wt = torch.from_numpy(w["wk"])
    exp_k = wt.reshape(cfg.n_kv_heads, d, H).repeat_interleave(rep, 0).reshape(cfg.n_q_heads * d, H).numpy()
    exp_v = torch.from_numpy(w["wv"]).reshape(cfg.n_kv_heads, d, H).repeat_interleave(rep, 0).reshape(cfg.n_q_heads * d, H).numpy()
    mha_cfg = vs.scaled(cfg, n_kv_heads=cfg.n_q_heads)
    w2 = dict(w, wk=exp_k, wv=exp_v)
    x = np.random.default_rng(16).standard_normal((cfg.seq, H))
    cos, sin = _text_tables(cfg.capacity, d, cfg.theta)
    kc = np.zeros((cfg.n_kv_heads, cfg.capacity, d)); vc = np.zeros_like(kc)
    kc2 = np.zeros((cfg.n_q_heads, cfg.capacity, d)); vc2 = np.zeros_like(kc2)
    a = od.decoder_layer(x, w, cfg, kc, vc, 0, cos, sin, od.F64)
    b = od.decoder_layer(x, w2, mha_cfg, kc2, vc2, 0, cos, sin, od.F64)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
    p = pages()["penguin_gqa_expand"]
    assert list(torch.zeros(p["kv_weight_shape"]).reshape(8, 128, 1024).repeat_interleave(p["repeat"], 0)
                .reshape(16 * 128, 1024).shape) == p["expanded_shape"]


def test_decoder_layer_causal():
    cfg = TINY
    w = {k: v.astype(np.float64) for k, v in vs.decoder_layer_weights(cfg, 0).items()}
    rng = np.random.default_rng(17)
    x = rng.standard_normal((cfg.seq, cfg.hidden))
    x2 = x.copy(); x2[3:] = rng.standard_normal((cfg.seq - 3, cfg.hidden))
    cos, sin = _text_tables(cfg.capacity, cfg.head_dim, cfg.theta)
    outs = []
    for xx in (x, x2):
        kc = np.zeros((2, cfg.capacity, 4)); vc = np.zeros_like(kc)
        outs.append(od.decoder_layer(xx, w, cfg, kc, vc, 0, cos, sin, od.F64))
    assert np.array_equal(outs[0][:3], outs[1][:3])


def test_bf16_mode_stays_close_to_f64():
    cfg = vs.scaled(TINY, dtype="bf16", hidden=64, head_dim=16, ffn=96)
    w = vs.decoder_layer_weights(cfg, 0)
    x = np.random.default_rng(18).standard_normal((cfg.seq, cfg.hidden))
    cos, sin = _text_tables(cfg.capacity, cfg.head_dim, cfg.theta)
    outs = []
    for prec in (od.BF16, od.F64):
        kc = np.zeros((2, cfg.capacity, 16)); vc = np.zeros_like(kc)
        ww = {k: (v if prec == od.BF16 else v.astype(np.float64)) for k, v in w.items()}
        outs.append(od.decoder_layer(x, ww, cfg, kc, vc, 0, cos, sin, prec))
        if prec == od.BF16:   # cached K/V are bf16 values
            assert np.array_equal(od.bf16_round(kc), kc) and np.array_equal(od.bf16_round(vc), vc)
    err = np.abs(outs[0] - outs[1]).max() / np.abs(outs[1]).max()
    assert 1e-5 < err < 2e-2


def _sharpened(w):
    """bf16 layer weights with every matrix scaled by 16 (still bf16 values): at
    the workloads' 0.02 scale a tiny layer's attention is nearly uniform, so a
    rounding of q can vanish under the later rounding of the attention output;
    larger weights make each rounding point visible."""
    return {k: v.astype(np.float64) * (16.0 if v.ndim == 2 else 1.0) for k, v in w.items()}


def _bf16_rounder(skip=None):
    """Storage rounding for the brute-force layers, optionally left out at one point."""
    return lambda vec, tag: list(vec) if tag == skip else [bf.bf16(t) for t in vec]


def test_bf16_round_agrees_with_bit_level_rounding():
    """Two independent roundings to bfloat16 (the oracle's frexp form and the
    brute-force bit-level form) agree on random values, exact ties and carries."""
    rng = np.random.default_rng(31)
    vals = np.r_[rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                 1.0 + (2 * np.arange(64) + 1) * 2.0 ** -9, 1.9999999, -3.99609375, 255.5]
    ref = od.bf16_round(vals)
    assert all(bf.bf16(float(v)) == float(r) for v, r in zip(vals, ref))


BF16_TAGS = ("h", "q", "k", "v", "o", "h2", "a")


@pytest.mark.parametrize("qk_norm", [1, 0])
def test_bf16_decoder_layer_rounding_points_match_brute_force(qk_norm):
    """Reading of the bf16 policy: the operands of every projection (normed
    rows, attention output, SwiGLU product), q and the cached k/v are stored
    as bf16; products are exact and summed exactly. The oracle's bf16 layer
    equals a pure-Python layer that rounds at exactly those points (fsum
    sums); leaving any one of the seven rounding points out of the brute
    force breaks the agreement of the layer output or of the cached K/V, so
    each point is pinned."""
    cfg = vs.scaled(TINY, dtype="bf16", hidden=16, head_dim=8, ffn=24, qk_norm=qk_norm)
    w = _sharpened(vs.decoder_layer_weights(cfg, 0))
    x = np.random.default_rng(32).standard_normal((cfg.seq, cfg.hidden))
    cos, sin = _text_tables(cfg.capacity, cfg.head_dim, cfg.theta)
    kc = np.zeros((cfg.n_kv_heads, cfg.capacity, cfg.head_dim)); vc = np.zeros_like(kc)
    got = od.decoder_layer(x, w, cfg, kc, vc, 0, cos, sin, od.BF16)
    rep = cfg.n_q_heads // cfg.n_kv_heads
    wl = {k: v.tolist() for k, v in w.items()}
    wl["wk"] = bf.expand_kv_rows(wl["wk"], cfg.n_kv_heads, cfg.head_dim, rep)
    wl["wv"] = bf.expand_kv_rows(wl["wv"], cfg.n_kv_heads, cfg.head_dim, rep)

    def brute(skip):
        ck, cv = [], []
        out = bf.decoder_layer_mha(x.tolist(), wl, cfg.n_q_heads, cfg.head_dim, cfg.eps, cfg.theta, qk_norm, 0,
                                   ck, cv, rnd=_bf16_rounder(skip))
        return np.asarray(out), ck, cv
    ref, ck, cv = brute(None)
    delta = np.abs(got - x).max()          # what the layer adds to the residual rows
    assert np.abs(got - ref).max() <= 1e-12 * delta
    for s in range(cfg.seq):
        for g in range(cfg.n_kv_heads):
            assert np.array_equal(kc[g, s], ck[s][g * rep]) and np.array_equal(vc[g, s], cv[s][g * rep])
    for tag in BF16_TAGS:   # observable in the layer output or in the cached K/V
        other, ok_, ov_ = brute(tag)
        moved = np.abs(other - got).max() > 1e-6 * delta
        moved |= any(not np.array_equal(kc[g, s], ok_[s][g * rep]) or not np.array_equal(vc[g, s], ov_[s][g * rep])
                     for s in range(cfg.seq) for g in range(cfg.n_kv_heads))
        assert moved, tag


def test_bf16_lm_head_rounds_the_final_row():
    rng = np.random.default_rng(33)
    E = np.asarray(vs.to_bf16_values(rng.standard_normal((9, 6)).astype(np.float32)), np.float64)
    x, g = rng.standard_normal(6), np.asarray(vs.to_bf16_values(rng.standard_normal(6).astype(np.float32)), np.float64)
    lg = od.lm_head_logits(x, g, E, 1e-6, od.BF16)
    row = [bf.bf16(t) for t in bf.rmsnorm(list(x), list(g), 1e-6)]
    assert np.allclose(lg, bf.matvec_exact(E.tolist(), row), rtol=1e-13, atol=1e-15)
    assert not np.allclose(lg, bf.matvec(E.tolist(), bf.rmsnorm(list(x), list(g), 1e-6)), rtol=1e-6)


def test_bf16_sum_modes_differ_only_by_summation_order():
    """BF16_F32SUM (float32 BLAS sums, the noise-floor probe) moves a layer by
    float32 rounding only; the exact mode equals the brute force above."""
    cfg = vs.scaled(TINY, dtype="bf16", hidden=64, head_dim=16, ffn=96)
    w = vs.decoder_layer_weights(cfg, 0)
    x = np.random.default_rng(34).standard_normal((cfg.seq, cfg.hidden))
    cos, sin = _text_tables(cfg.capacity, cfg.head_dim, cfg.theta)
    outs = []
    for prec in (od.BF16, od.BF16_F32SUM):
        kc = np.zeros((2, cfg.capacity, 16)); vc = np.zeros_like(kc)
        outs.append(od.decoder_layer(x, w, cfg, kc, vc, 0, cos, sin, prec))
    err = np.abs(outs[0] - outs[1]).max() / np.abs(outs[0]).max()
    assert err < 2e-2


def test_bf16_vit_layer_rounding_points_match_brute_force():
    """The bf16-storage vision layer (HunyuanOCR v1.5 port §3.7, Mixed policy)
    rounds at the same kinds of points as the decoder (tags h, q, k, v, o, h2 and
    the GELU output f); each point pinned as in the decoder test."""
    cfg = vs.scaled_vit(TINY_VIT, dtype="bf16")
    w = _sharpened(vs.vit_layer_weights(cfg, 0))
    x = np.random.default_rng(35).standard_normal((cfg.n_patches, cfg.hidden))
    pos = ov.vit_positions(cfg)
    axes = np.r_[np.zeros(1, np.int64), np.ones(1, np.int64)]
    cos, sin = od.rope_tables(pos, axes, 2, cfg.head_dim, cfg.theta)
    seg = (pos[0] // 4) * 10 + pos[1] // 4
    mask = np.where(seg[:, None] == seg[None, :], 0.0, od.MASK_NEG)
    got = ov.vit_layer(x, w, mask, cos, sin, cfg, od.BF16)
    wl = {k: v.tolist() for k, v in w.items()}

    def brute(skip):
        return np.asarray(bf.vit_layer(x.tolist(), wl, cfg.n_heads, cfg.head_dim, cfg.eps, pos.tolist(), cfg.theta,
                                       lambda i, j: seg[i] == seg[j], rnd=_bf16_rounder(skip)))
    delta = np.abs(got - x).max()
    assert np.abs(got - brute(None)).max() <= 1e-12 * delta
    for tag in ("h", "q", "k", "v", "o", "h2", "f"):
        assert np.abs(brute(tag) - got).max() > 1e-6 * delta, tag


def test_vit_bf16_mode_stays_close_to_f64():
    """The vision tower's bf16-storage mode (HunyuanOCR v1.5 port §3.7 Mixed policy) moves the
    merged rows by bf16 rounding only: same bf16-valued weights, the two rounding modes differ by
    more than float noise and by less than the bf16 gate."""
    cfgb = vs.scaled_vit(vs.C5, n_layers=2, full_layers=(1,), grid_h=4, grid_w=8, window=2, dtype="bf16")
    glob = vs.vit_globals(cfgb)
    layers = [vs.vit_layer_weights(cfgb, l) for l in range(cfgb.n_layers)]
    rb = ov.run_vit(cfgb, glob, layers)["out"]
    rf = ov.run_vit(vs.scaled_vit(cfgb, dtype="f32"), glob, layers)["out"]
    err = np.abs(rb - rf).max() / np.abs(rf).max()
    assert 1e-5 < err < 2e-2


# ----------------------------------------------------------------------------- whole decoder
def _tiny_run(cfg, **kw):
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    return od.run_decoder(cfg, glob, layers, **kw), glob, layers


def test_prefill_equals_decode_replay():
    """Youtu-VL ncnn port, 结果展示: decode replay of the prompt reproduces the
    parallel prefill (3.0e-7 relative there in fp32); in float64 the oracle's
    two paths agree to rounding."""
    cfg = vs.scaled(vs.C1, seq=12, n_img=4, img_start=3, decode_steps=4, capacity=20, n_layers=2)
    a, _, _ = _tiny_run(cfg)
    b, _, _ = _tiny_run(cfg, prefill_split=5)
    rel = np.abs(a["prefill_x"] - b["prefill_x"]).max() / np.abs(a["prefill_x"]).max()
    assert rel < 1e-12 < pages()["youtu_replay_rel_error"]["value"]
    assert np.allclose(a["logits0"], b["logits0"], rtol=1e-11, atol=1e-12)
    assert list(a["ids"]) == list(b["ids"])
    T = cfg.seq + cfg.decode_steps
    assert np.allclose(a["k_cache"][:, :, :T], b["k_cache"][:, :, :T], rtol=1e-11, atol=1e-13)


def test_block_logits_equal_decode_steps():
    """The verify head's definition (one causal forward over prompt + block, a head on every
    block row) gives the logits of one-token decode steps fed the same tokens (the pages'
    prefill = decode replay, HunyuanOCR v1.5 port §3.8 for the verify use)."""
    cfg = vs.scaled(vs.C1, seq=12, n_img=4, img_start=3, decode_steps=5, capacity=20, n_layers=2)
    a, glob, layers = _tiny_run(cfg, keep_logits=True)
    block = [int(i) for i in a["ids"][:5]]
    got = od.block_logits(cfg, glob, layers, block)
    want = np.stack(a["step_logits"])
    assert np.allclose(got, want, rtol=1e-11, atol=1e-12)
    assert [int(np.argmax(r)) for r in got] == [int(i) for i in a["ids"][1:6]]


def test_hidden_state_decode_equals_longer_prefill():
    """A stack without vocabulary decodes given rows: the hidden output of decode step i equals
    the prefill output of the same row appended to the prompt (prefill = decode replay)."""
    cfg = vs.scaled(vs.C2_F32, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=64, seq=6, decode_steps=3,
                    capacity=12)
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    a = od.run_decoder(cfg, glob, layers)
    cfg9 = vs.scaled(cfg, seq=9, decode_steps=0)
    b = od.run_decoder(cfg9, dict(glob, x=np.concatenate([glob["x"], glob["decode_x"]])), layers)
    assert np.allclose(a["decode_x"], b["prefill_x"][6:], rtol=1e-11, atol=1e-12)


def test_cache_after_short_prefill_is_prefix_of_long_prefill():
    cfg = vs.scaled(vs.C1, seq=10, n_img=2, img_start=2, decode_steps=0, capacity=16)
    a, glob, layers = _tiny_run(cfg)
    cfg6 = vs.scaled(cfg, seq=6)
    glob6 = dict(glob, ids=glob["ids"][:6])
    b = od.run_decoder(cfg6, glob6, layers, steps=0)
    # equal up to BLAS blocking order (the row count differs between the two runs)
    assert np.allclose(a["k_cache"][:, :, :6], b["k_cache"][:, :, :6], rtol=1e-12, atol=1e-14)
    assert np.allclose(a["v_cache"][:, :, :6], b["v_cache"][:, :, :6], rtol=1e-12, atol=1e-14)
    assert not np.allclose(a["k_cache"][:, :, 6:10], 0)


def test_decode_step_uses_previous_token_embedding():
    cfg = vs.scaled(vs.C1, seq=8, n_img=2, img_start=2, decode_steps=2, capacity=16)
    a, glob, layers = _tiny_run(cfg)
    # re-run with the first generated id appended to the prompt: its prefill logits = step-1 logits
    cfg9 = vs.scaled(cfg, seq=9, decode_steps=0)
    glob9 = dict(glob, ids=np.r_[glob["ids"], a["ids"][0]].astype(np.int32))
    b = od.run_decoder(cfg9, glob9, layers, steps=0)
    assert b["ids"][0] == a["ids"][1]


def test_capacity_rejected():
    cfg = vs.scaled(vs.C1, seq=10, n_img=2, img_start=2, decode_steps=8, capacity=16)
    with pytest.raises(ValueError):
        _tiny_run(cfg)


# ----------------------------------------------------------------------------- ViT
def test_vit_window_counts_match_page():
    p = pages()
    cfg = vs.C5
    assert (cfg.grid_h, cfg.grid_w) == (p["youtu_grid"]["grid_h"], p["youtu_grid"]["grid_w"])
    assert cfg.n_patches == p["youtu_grid"]["patches"] and cfg.n_merged == p["youtu_grid"]["merged_tokens"]
    assert cfg.hidden * 4 == p["youtu_vision"]["merge_concat_width"] and cfg.out_dim == p["youtu_vision"]["merger_out"]
    assert tuple(p["youtu_vision"]["full_attention_layers"]) == cfg.full_layers
    perm, seg = ov.vit_window_order(cfg)
    assert sorted(perm) == list(range(322))
    sizes = np.bincount(seg) * 4
    assert list(sizes) == [224, 224, 224, 224, 224, 168]
    assert np.all(np.diff(seg) >= 0)        # windows contiguous after permutation
    pos = ov.vit_positions(cfg)
    assert len({(h, w) for h, w in pos.T}) == 1288
    assert pos[0].max() == 13 and pos[1].max() == 91
    u = 46 * 3 + 5                          # merge unit (3, 5) holds patches (6..7, 10..11)
    assert {tuple(pos[:, 4 * u + i]) for i in range(4)} == {(6, 10), (6, 11), (7, 10), (7, 11)}


def test_other_page_counts():
    p = pages()
    assert p["penguin_patches"]["grid"][0] * p["penguin_patches"]["grid"][1] == p["penguin_patches"]["patches"] == vs.C3.n_img
    h, w = p["hunyuan_v10_span"]["h"], p["hunyuan_v10_span"]["w"]
    assert 1 + h * (w + 1) + 1 == p["hunyuan_v10_span"]["rows"]
    gh, gw = p["hunyuan_v15_tokens"]["grid"]; m = p["hunyuan_v15_tokens"]["merge"]
    assert (gh // m) * (gw // m + 1) + 2 == p["hunyuan_v15_tokens"]["tokens"]
    q = p["penguin_qwen3"]
    assert (vs.C3.hidden, vs.C3.n_layers, vs.C3.n_q_heads, vs.C3.n_kv_heads, vs.C3.head_dim, vs.C3.vocab) == \
        (q["hidden"], q["layers"], q["q_heads"], q["kv_heads"], q["head_dim"], q["vocab"])


TINY_VIT = vs.VitConfig("tiny_vit", 98, n_layers=2, hidden=8, n_heads=2, head_dim=4, ffn=12, grid_h=4, grid_w=6,
                        merge=2, window=2, full_layers=(1,), merger_hidden=10, out_dim=6, theta=1e4)


def test_vit_layer_matches_brute_force():
    cfg = TINY_VIT
    w = {k: v.astype(np.float64) for k, v in vs.vit_layer_weights(cfg, 0).items()}
    x = np.random.default_rng(19).standard_normal((cfg.n_patches, cfg.hidden))
    pos = ov.vit_positions(cfg)
    axes = np.r_[np.zeros(1, np.int64), np.ones(1, np.int64)]
    cos, sin = od.rope_tables(pos, axes, 2, cfg.head_dim, cfg.theta)
    seg = (pos[0] // 4) * 10 + pos[1] // 4      # arbitrary window ids
    mask = np.where(seg[:, None] == seg[None, :], 0.0, od.MASK_NEG)
    got = ov.vit_layer(x, w, mask, cos, sin, cfg)
    ref = bf.vit_layer(x.tolist(), {k: v.tolist() for k, v in w.items()}, cfg.n_heads, cfg.head_dim, cfg.eps,
                       pos.tolist(), cfg.theta, lambda i, j: seg[i] == seg[j])
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_vit_permutation_is_undone():
    """With every layer full-attention the tower is permutation-equivariant, so
    the window permutation must cancel: compare with an unpermuted run."""
    cfg = vs.scaled_vit(TINY_VIT, full_layers=(0, 1))
    glob = vs.vit_globals(cfg)
    layers = [vs.vit_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    res = ov.run_vit(cfg, glob, layers)
    x = glob["x"].astype(np.float64)
    pos = ov.vit_positions(cfg)
    axes = np.r_[np.zeros(1, np.int64), np.ones(1, np.int64)]
    cos, sin = od.rope_tables(pos, axes, 2, cfg.head_dim, cfg.theta)
    for w in layers:
        x = ov.vit_layer(x, {k: v.astype(np.float64) for k, v in w.items()}, np.zeros((24, 24)), cos, sin, cfg)
    g = {k: v.astype(np.float64) for k, v in glob.items()}
    z = od.layer_norm(x, g["post_ln"], g["post_ln_b"], cfg.eps).reshape(cfg.n_merged, 4 * cfg.hidden)
    y = od.gelu_tanh(z @ g["m1"].T + g["m1b"]) @ g["m2"].T + g["m2b"]
    assert np.allclose(res["out"], y, rtol=1e-11, atol=1e-12)


def test_vit_window_attention_is_per_window():
    cfg = TINY_VIT
    perm, seg = ov.vit_window_order(cfg)
    rows = np.repeat(seg, 4)
    rng = np.random.default_rng(20)
    q, k, v = (rng.standard_normal((2, len(rows), 4)) for _ in range(3))
    mask = np.where(rows[:, None] == rows[None, :], 0.0, od.MASK_NEG)
    full = od.softmax_attention(q, k, v, mask, 1)
    for wid in np.unique(rows):
        sel = rows == wid
        n = sel.sum()
        part = od.softmax_attention(q[:, sel], k[:, sel], v[:, sel], np.zeros((n, n)), 1)
        assert np.allclose(full[:, sel], part, rtol=1e-14, atol=1e-15)
