"""GPU parity of the expanded multi-head latent attention stack (block_kind MLA)
against the oracle, through the C ABI.

The layer is the one the Youtu-VL-4B ncnn port runs (实现流程 §6): the
512-wide compressed KV is expanded per head by kv_b, the cache holds keys 192
wide (128 + 64 rotated, interleaved RoPE per 实现难点 §2) and values 128 wide,
and every query head has its own KV head. The stack is cut to 4 heads and
hidden 512 so the oracle finishes in seconds; the head shapes are the pages'.
Checks: prefill rows, first-token logits, K and V caches after the prefill and
after the decode steps, greedy ids; chunked prefill equals one prefill.
Gates as for the other stacks: 1e-4 (fp32), 2e-2 (bf16), ids exact for fp32
and with near-tie attribution for bf16.
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
        assert k.shape[-1] == cfg.head_dim and v.shape[-1] == cfg.v_head_dim
        assert rel(k[:, :T], ref["k_cache"][l][:, :T]) <= tol, f"layer {l} K"
        assert rel(v[:, :T], ref["v_cache"][l][:, :T]) <= tol, f"layer {l} V"


def test_mla_f32_end_to_end(pipeline):
    cfg = vs.C_MLA
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


def test_mla_f32_chunked_prefill_equals_full(pipeline):
    cfg = vs.C_MLA
    glob, layers = make(cfg)
    a = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    xa = a.prefill().cpu().numpy()
    b = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    b.embed_inject()
    for p0, s in ((0, 20), (20, 17), (37, cfg.seq - 37)):
        b.model.prefill(b.x[p0:p0 + s], p0, b.cos, b.sin, [pipeline.causal_mask()], b.kv, b.ws)
    assert b.kv.len() == cfg.seq
    assert rel(b.x.cpu().numpy(), xa) <= 1e-5
    for l in range(cfg.n_layers):
        ka, va = kv_host(a, l)
        kb, vb = kv_host(b, l)
        assert rel(kb[:, :cfg.seq], ka[:, :cfg.seq]) <= 1e-5 and rel(vb[:, :cfg.seq], va[:, :cfg.seq]) <= 1e-5


def test_mla_bf16_end_to_end(pipeline):
    cfg = vs.scaled(vs.C_MLA, dtype="bf16", decode_steps=12)
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
    check_caches(run, ref, cfg, cfg.seq + cfg.decode_steps, TOL["bf16"])
    run.kv.truncate(cfg.seq)
    forced = [tok0] + list(run.decode_forced(ref["ids"][:-1]))
    print(f"mla bf16: first-token logit err {np.abs(lg - ref['logits0']).max():.2e}")
    check_ids("mla bf16", free, forced, ref["ids"], ref["margins"], ref["floor"])


def test_mla_bf16_few_row_chunks_match_oracle(pipeline):
    """bf16 expanded-MLA stack prefilled in chunks of 16, 1, 7 and 8 rows after a 16-row first chunk
    (every projection of the chunks, the latent ones with K = 512 included, on the few-row path, and the
    attention of 1-16 query rows per head on the few-row launch): hidden rows and the K/V caches against
    the oracle's one-shot prefill within the 2e-2 bf16 gate."""
    cfg = vs.scaled(vs.C_MLA, dtype="bf16", decode_steps=0)
    glob, layers = make(cfg)
    ref = od.run_decoder(cfg, glob, layers, steps=0)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.embed_inject()
    p0 = 0
    for s in (16, 16, 1, 7, 8):
        s = min(s, cfg.seq - p0)
        run.model.prefill(run.x[p0:p0 + s], p0, run.cos, run.sin, [pipeline.causal_mask()], run.kv, run.ws)
        p0 += s
    if p0 < cfg.seq:
        run.model.prefill(run.x[p0:cfg.seq], p0, run.cos, run.sin, [pipeline.causal_mask()], run.kv, run.ws)
    assert run.kv.len() == cfg.seq
    assert rel(run.x.cpu().numpy(), ref["prefill_x"]) <= TOL["bf16"]
    check_caches(run, ref, cfg, cfg.seq, TOL["bf16"])
