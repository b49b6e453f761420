"""GPU parity of the decoder layer variants against the oracle, through the C ABI.

* QK-Norm after RoPE, with the cache holding the normalised k (HunyuanOCR
  v1.0 ncnn port, 二 and 五.2): desc.qk_norm = 2.
* Interleaved RoPE, adjacent pairs rotated and de-interleaved into the
  rotate-half order (Youtu-VL-4B ncnn port, 实现难点 §2): desc.rope_interleave = 1.

Both change the prefill RoPE kernel and the rotation inside the fused decode
attention, so every case checks the prefill rows, the K/V cache after the
prefill and after the decode steps, and the decode output. Gates as in the
other parity tests: 1e-4 relative for fp32, 2e-2 for bf16, ids exact (fp32)
or with near-tie attribution (bf16).
"""
import numpy as np
import pytest
import torch

from oracle import decoder as od
import vlm_synth as vs
from tests._parity import check_ids, oracle_run
from tests.test_gpu_decoder import TOL, kv_host, make, rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pipeline():
    from decoder_prefill_decode_amd import pipeline
    return pipeline


def check_caches(run, ref, cfg, T, tol):
    for l in range(cfg.n_layers):
        k, v = kv_host(run, l)
        assert rel(k[:, :T], ref["k_cache"][l][:, :T]) <= tol, f"layer {l} K"
        assert rel(v[:, :T], ref["v_cache"][l][:, :T]) <= tol, f"layer {l} V"


@pytest.mark.parametrize("qk_norm,interleave", [(2, False), (0, True), (2, True), (1, True)],
                         ids=["norm_after", "interleave", "norm_after_interleave", "norm_before_interleave"])
def test_f32_stack_variants(pipeline, qk_norm, interleave):
    cfg = vs.scaled(vs.C1, qk_norm=qk_norm, rope_interleave=interleave)
    glob, layers = make(cfg)
    ref = od.run_decoder(cfg, glob, layers)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    x = run.prefill()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    tok0 = int(run.first_token(logits)[0])
    assert rel(x.cpu().numpy(), ref["prefill_x"]) <= TOL["f32"]
    assert rel(logits.cpu().numpy(), ref["logits0"]) <= TOL["f32"]
    check_caches(run, ref, cfg, cfg.seq, TOL["f32"])
    ids = run.decode(cfg.decode_steps, loop=True)
    assert [tok0] + list(ids) == list(ref["ids"])
    check_caches(run, ref, cfg, cfg.seq + cfg.decode_steps, TOL["f32"])


def test_bf16_layer_norm_after_interleave(pipeline):
    cfg = vs.scaled(vs.C2_BF16, qk_norm=2, rope_interleave=True, seq=200, decode_steps=24, capacity=256)
    glob, layers = make(cfg)
    ref = od.run_decoder(cfg, glob, layers)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    x = run.prefill()
    assert rel(x.cpu().numpy(), ref["prefill_x"]) <= TOL["bf16"]
    check_caches(run, ref, cfg, cfg.seq, TOL["bf16"])
    out = run.decode_hidden(run.dec_x).cpu().numpy()
    assert rel(out, ref["decode_x"]) <= TOL["bf16"]
    check_caches(run, ref, cfg, cfg.seq + cfg.decode_steps, TOL["bf16"])


def test_bf16_head80_stack_interleave(pipeline):
    """80-wide heads (40 rotation pairs, 4 query heads per KV head) with interleaved RoPE and QK-Norm after it."""
    cfg = vs.scaled(vs.C4, n_layers=2, vocab=8192, seq=80, n_img=30, img_start=16, decode_steps=12, capacity=128,
                    qk_norm=2, rope_interleave=True)
    glob, layers = make(cfg)
    ref = oracle_run(cfg, glob, layers)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    x = run.prefill()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    tok0 = int(run.first_token(logits)[0])
    lg = logits.cpu().numpy()
    assert rel(x.cpu().numpy(), ref["prefill_x"]) <= TOL["bf16"]
    assert rel(lg, ref["logits0"]) <= TOL["bf16"]
    check_caches(run, ref, cfg, cfg.seq, TOL["bf16"])
    free = [tok0] + list(run.decode(cfg.decode_steps))
    run.kv.truncate(cfg.seq)
    forced = [tok0] + list(run.decode_forced(ref["ids"][:-1]))
    print(f"head80 variants: first-token logit err {np.abs(lg - ref['logits0']).max():.2e}")
    check_ids("head80 variants", free, forced, ref["ids"], ref["margins"], ref["floor"])


# (head_dim, n_q_heads, n_kv_heads): groups of 8 and 4 query heads per KV head at widths 64, 80, 128
GROUP_SHAPES = [(64, 16, 2), (80, 32, 4), (128, 16, 4), (64, 8, 2), (128, 32, 4)]


def group_stack(hd, nq, nkv):
    """One bf16 layer with a 180-row prompt (its last 16-key tile ragged) and 24 decode steps that
    cross the split plan's band boundary at position 192."""
    return vs.scaled(vs.C2_BF16, hidden=512, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd, ffn=1024, seq=180,
                     decode_steps=24, capacity=256)


@pytest.mark.parametrize("hd,nq,nkv", GROUP_SHAPES, ids=["d64_g8", "d80_g8", "d128_g4", "d64_g4", "d128_g8"])
def test_bf16_decode_groups_of_4_and_8(pipeline, hd, nq, nkv):
    """bf16 decode with 4 or 8 query heads per KV head (scored on the matrix cores): prefill rows,
    decode hidden rows and both caches against the oracle at the bf16 gate."""
    cfg = group_stack(hd, nq, nkv)
    glob, layers = make(cfg)
    ref = od.run_decoder(cfg, glob, layers)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    x = run.prefill()
    assert rel(x.cpu().numpy(), ref["prefill_x"]) <= TOL["bf16"]
    out = run.decode_hidden(run.dec_x).cpu().numpy()
    assert rel(out, ref["decode_x"]) <= TOL["bf16"]
    check_caches(run, ref, cfg, cfg.seq + cfg.decode_steps, TOL["bf16"])


@pytest.mark.parametrize("splits", [32, 1], ids=["plan", "one_split"])
@pytest.mark.parametrize("hd,nq,nkv", GROUP_SHAPES[:3], ids=["d64_g8", "d80_g8", "d128_g4"])
def test_matrix_core_decode_attention_equals_vector_form(pipeline, monkeypatch, hd, nq, nkv, splits):
    """The matrix-core decode attention (VLM_DEC_MFMA unset) against the vector-ALU form
    (VLM_DEC_MFMA=0) on the same prompt and steps: caches bitwise equal (both write the same rotated
    k / v), hidden rows within 1e-3 (P enters the P.V products as a bf16 hi + lo pair). One split
    gives each wavefront 3-4 tiles, two batches, so the online rescale between batches runs."""
    cfg = group_stack(hd, nq, nkv)
    glob, layers = make(cfg)
    monkeypatch.setenv("VLM_DEC_SPLITS", str(splits))
    outs, caches = [], []
    for form in ("1", "0"):
        monkeypatch.setenv("VLM_DEC_MFMA", form)
        run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
        run.prefill()
        outs.append(run.decode_hidden(run.dec_x).cpu().numpy())
        caches.append(kv_host(run, 0))
        del run
    T = cfg.seq + cfg.decode_steps
    for a, b in zip(caches[0], caches[1]):
        assert np.array_equal(a[:, :T], b[:, :T])
    err = rel(outs[0], outs[1])
    print(f"d{hd} g{nq // nkv} splits {splits}: matrix-core vs vector form {err:.2e}")
    assert err <= 1e-3


def test_deep_gemm_ring_equals_two_stage_ring(pipeline, monkeypatch):
    """The prefill GEMMs' deeper LDS rings (default) against the shallow ones (VLM_LDS_DEEP=0) on
    the tile shapes that take them: a 2-layer bf16 vision tower at full width (128x192 QKV and fc1,
    64x128 O, 128x256 split fc2; one window and one full-attention layer) and a one-layer prefill at
    the 36-layer stack's width (64x128 QKV, 128x128 split O, 128x256 split down). Only the number of
    stages in flight differs, so the outputs are bitwise equal."""
    vcfg = vs.scaled_vit(vs.C5, dtype=vs.BF16, n_layers=2, full_layers=(1,), name="c5_vit_2l_bf16")
    vglob = vs.vit_globals(vcfg)
    dcfg = vs.scaled(vs.C4, n_layers=1, vocab=4096, name="c4_1l")
    glob, layers = make(dcfg)
    outs = {}
    for deep in ("1", "0"):
        monkeypatch.setenv("VLM_LDS_DEEP", deep)
        run = pipeline.VitRun(vcfg, lambda l: vs.vit_layer_weights(vcfg, l), vglob)
        v = run.run().cpu().numpy()
        del run
        drun = pipeline.DecoderRun(dcfg, lambda l: layers[l], glob)
        x = drun.prefill().cpu().numpy()
        del drun
        outs[deep] = (v, x)
    assert np.isfinite(outs["1"][0]).all() and np.isfinite(outs["1"][1]).all()
    assert np.array_equal(outs["1"][0], outs["0"][0])
    assert np.array_equal(outs["1"][1], outs["0"][1])
