"""Multi-token verify and commit (HunyuanOCR v1.5 ncnn port §3.8: the target model
verifies a drafted block in one causal forward, keeps the longest matching
prefix plus its first correction, and trims the caches).

fp32 4B-class layer shape (2 layers, vocab 8192), whose greedy sequence varies:
  * the verify head's logits of a block equal the oracle's by definition (one
    causal forward over prompt + block) within 1e-4, its picks are the
    oracle's greedy ids;
  * drafting from the greedy sequence with wrong tokens injected at chosen
    positions, verify + commit reproduces the one-token decode's ids exactly
    and leaves the same cache (1e-4) and length.
"""
import numpy as np
import pytest
import torch

from oracle import decoder as od
import vlm_synth as vs
from tests._parity import rel

pytestmark = pytest.mark.gpu

CFG = vs.scaled(vs.C4, n_layers=2, vocab=8192, seq=80, n_img=30, img_start=16, decode_steps=40, capacity=128,
                dtype="f32", name="c4_2layer_f32_verify")


@pytest.fixture(scope="module")
def env():
    from decoder_prefill_decode_amd import pipeline
    glob = vs.decoder_globals(CFG)
    layers = [vs.decoder_layer_weights(CFG, l) for l in range(CFG.n_layers)]
    ref = od.run_decoder(CFG, glob, layers, steps=CFG.decode_steps + 8)   # ids past the last step for drafts
    return pipeline, glob, layers, [int(i) for i in ref["ids"]]


def test_verify_head_matches_causal_forward(env):
    pipeline, glob, layers, ids = env
    k = 8
    block = ids[:k]
    want = od.block_logits(CFG, glob, layers, block)
    run = pipeline.DecoderRun(CFG, lambda l: layers[l], glob)
    run.prefill()
    assert int(run.first_token()[0]) == ids[0]
    logits = torch.empty((k, CFG.vocab), dtype=torch.float32, device="cuda")
    toks, nxt = run.verify_block(block, logits)
    assert rel(logits.cpu().numpy(), want) <= 1e-4
    assert [int(np.argmax(r)) for r in want] == ids[1:k + 1]
    assert toks == ids[1:k + 1] and nxt == ids[k]          # every draft accepted, plus the next token
    assert run.kv.len() == CFG.seq + k


@pytest.mark.parametrize("k,wrong", [(6, {1: [3], 2: [1], 4: [5], 5: [1, 2]}), (4, {0: [1], 3: [2]})],
                         ids=["block6", "block4"])
def test_draft_accept_commit_reproduces_greedy_decode(env, k, wrong):
    """wrong: {block number: block offsets whose drafted token is replaced by another id}."""
    pipeline, glob, layers, ids = env
    N = CFG.decode_steps
    ar = pipeline.DecoderRun(CFG, lambda l: layers[l], glob)
    ar.prefill()
    t0 = int(ar.first_token()[0])
    ar_ids = [t0] + [int(t) for t in ar.decode(N)]
    assert ar_ids == ids[:N + 1]
    T = CFG.seq + N

    sp = pipeline.DecoderRun(CFG, lambda l: layers[l], glob)
    sp.prefill()
    gen = [int(sp.first_token()[0])]
    blocks = 0
    while len(gen) < N + 1:
        i0 = len(gen) - 1                                   # gen[-1] == ids[i0], not yet in the cache
        draft = [gen[-1]] + ids[i0 + 1:i0 + k]
        for off in wrong.get(blocks, []):
            if off < k:
                draft[off] = (draft[off] + 1) % (CFG.vocab - 1)
        pos0 = sp.kv.len()
        assert pos0 == CFG.seq + i0
        toks, _ = sp.verify_block(draft)
        bad = [off for off in range(1, k) if draft[off] != ids[i0 + off]]
        expect_acc = (bad[0] - 1) if bad else k - 1         # drafted tokens before the first wrong one
        assert len(toks) == expect_acc + 1 and sp.kv.len() == pos0 + expect_acc + 1
        gen += toks
        blocks += 1
    assert gen[:N + 1] == ids[:N + 1]
    assert blocks < N                                       # fewer target passes than one-token decode
    assert sp.kv.len() >= T
    for l in range(CFG.n_layers):
        ka, va = (t[:, :T].cpu().numpy() for t in ar.kv.kv(l))
        kb, vb = (t[:, :T].cpu().numpy() for t in sp.kv.kv(l))
        assert rel(kb, ka) <= 1e-4 and rel(vb, va) <= 1e-4
    print(f"block {k}: {N + 1} greedy ids reproduced in {blocks} verify passes")


def test_verify_head_without_logits_buffer_beyond_the_split_scratch():
    """The verify head with its logits in the workspace, for a vocabulary wider than four times every row
    width of the stack (16384 > 4 x 1536 on the tiny stack): picks equal the argmax of the oracle's block
    logits, row for row."""
    from decoder_prefill_decode_amd import pipeline
    cfg = vs.scaled(vs.C1, vocab=16384, decode_steps=8, name="c1_vocab16k")
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    block = [int(i) for i in np.random.default_rng(3).integers(0, cfg.vocab - 1, size=8)]
    want = [int(np.argmax(r)) for r in od.block_logits(cfg, glob, layers, block)]
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.prefill()
    pos0 = run.kv.len()
    ids = torch.tensor(block, dtype=torch.int32, device="cuda")
    xb = torch.empty((len(block), cfg.hidden), dtype=torch.float32, device="cuda")
    run.model.embed_ids(ids, xb)
    run.model.prefill(xb, pos0, run.cos, run.sin, pipeline.causal_mask(), run.kv, run.ws)
    pred = torch.empty(len(block), dtype=torch.int32, device="cuda")
    run.model.lmhead_argmax_rows(xb, pred, run.ws)      # no logits buffer
    assert [int(p) for p in pred.cpu()] == want



# ------------------------------------------------------------- bf16: projections of a few rows
BF16_CHUNKS = [
    vs.scaled(vs.C4, n_layers=2, vocab=4096, seq=60, n_img=20, img_start=8, decode_steps=0, capacity=96,
              name="c4_2layer_bf16_chunks"),
    vs.scaled(vs.C3, n_layers=2, vocab=4096, seq=60, n_img=20, img_start=8, decode_steps=0, capacity=96,
              name="c3_2layer_bf16_chunks"),
]


@pytest.mark.parametrize("cfg", BF16_CHUNKS, ids=lambda c: c.name)
def test_few_row_chunks_bf16_match_oracle(cfg):
    """bf16 chunked prefill in blocks of 1, 7 and 16 rows after a 36-row prefill (the blocks take the
    few-row projections: K split over 4, 8 and 16 wavefronts across the two layer shapes): hidden rows
    and both layers' K/V against the oracle's one-shot prefill within the 2e-2 bf16 gate."""
    from decoder_prefill_decode_amd import pipeline
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    ref = od.run_decoder(cfg, glob, layers, steps=0)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.embed_inject()
    for p0, s in ((0, 36), (36, 1), (37, 7), (44, 16)):
        run.model.prefill(run.x[p0:p0 + s], p0, run.cos, run.sin, [pipeline.causal_mask()], run.kv, run.ws)
    assert run.kv.len() == cfg.seq
    x = run.x.cpu().numpy()
    assert rel(x[36:], ref["prefill_x"][36:]) <= 2e-2
    assert rel(x, ref["prefill_x"]) <= 2e-2
    for l in range(cfg.n_layers):
        k, v = (t[:, :cfg.seq].float().cpu().numpy() for t in run.kv.kv(l))
        assert rel(k, ref["k_cache"][l][:, :cfg.seq]) <= 2e-2
        assert rel(v, ref["v_cache"][l][:, :cfg.seq]) <= 2e-2


def test_verify_head_bf16_matches_causal_forward():
    """bf16 4B-class shape: an 8-row verify block (few-row projections and the few-row lm_head) against
    the oracle's causal forward over prompt + block: logits within 2e-2, and every row whose top-2
    margin exceeds the oracle's own noise floor (float32 instead of exact sums) picks the oracle's id."""
    from decoder_prefill_decode_amd import pipeline
    cfg = vs.scaled(vs.C4, n_layers=2, vocab=8192, seq=60, n_img=20, img_start=8, decode_steps=8, capacity=96,
                    name="c4_2layer_bf16_verify")
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    block = [int(i) for i in np.random.default_rng(5).integers(0, cfg.vocab - 1, size=8)]
    want = od.block_logits(cfg, glob, layers, block)
    floor = float(np.abs(want - od.block_logits(cfg, glob, layers, block, prec=od.BF16_F32SUM)).max())
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.prefill()
    pos0 = run.kv.len()
    ids = torch.tensor(block, dtype=torch.int32, device="cuda")
    xb = torch.empty((len(block), cfg.hidden), dtype=torch.float32, device="cuda")
    run.model.embed_ids(ids, xb)
    run.model.prefill(xb, pos0, run.cos, run.sin, pipeline.causal_mask(), run.kv, run.ws)
    pred = torch.empty(len(block), dtype=torch.int32, device="cuda")
    logits = torch.empty((len(block), cfg.vocab), dtype=torch.float32, device="cuda")
    run.model.lmhead_argmax_rows(xb, pred, run.ws, logits)
    lg = logits.cpu().numpy()
    assert rel(lg, want) <= 2e-2
    top2 = np.sort(want, axis=1)[:, -2:]
    decided = [i for i in range(len(block)) if top2[i, 1] - top2[i, 0] > floor]
    print(f"verify head bf16: max logit error {np.abs(lg - want).max():.3e}, noise floor {floor:.3e}, "
          f"{len(decided)}/{len(block)} rows decided")
    assert [int(pred[i]) for i in decided] == [int(np.argmax(want[i])) for i in decided]
    assert [int(p) for p in pred.cpu()] == [int(np.argmax(r)) for r in lg]


@pytest.mark.parametrize("base", BF16_CHUNKS, ids=lambda c: c.name)
def test_few_row_attention_equals_row_tiled_attention(base, monkeypatch):
    """One bf16 layer, chunks of 1, 5, 8 and 16 rows at positions past a 150-row prefill (three to
    five 64-key tiles, causal): the few-row attention launch (the query heads of a KV head packed
    into one tile, key tiles split over blocks, merged by the decode merge kernel) against the
    row-tiled prefill attention on the same q, k and v (the projections are the few-row ones in
    both runs). The two differ only in summation order, so the layer outputs agree to 1e-3 of
    their scale, while a key seen past its row's position moves them by ~1e-2."""
    from decoder_prefill_decode_amd import pipeline
    cfg = vs.scaled(base, n_layers=1, seq=180, n_img=40, img_start=20, capacity=256, name=base.name + "_1layer")
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, 0)]
    outs = []
    for flag in ("3", "1"):
        monkeypatch.setenv("VLM_FEW_ROWS", flag)
        run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
        run.embed_inject()
        p0 = 150
        run.model.prefill(run.x[:p0], 0, run.cos, run.sin, [pipeline.causal_mask()], run.kv, run.ws)
        for s in (1, 5, 8, 16):
            run.model.prefill(run.x[p0:p0 + s], p0, run.cos, run.sin, [pipeline.causal_mask()], run.kv, run.ws)
            p0 += s
        outs.append(run.x[150:p0].cpu().numpy().copy())
    err = rel(outs[0], outs[1])
    print(f"{cfg.name}: few-row vs row-tiled attention, layer output max rel diff {err:.2e}")
    assert err <= 1e-3


def test_few_row_tails_bf16_match_oracle():
    """bf16 Qwen3 layer shape with a 4101-entry vocabulary (the verify head's table rows end 5 rows into
    a 16-row block) and chunks of 3, 12 and 2 rows (operand rows padded to 4 and 16): hidden rows and
    K/V against the oracle's one-shot prefill, and the head over the last chunk's rows against the
    oracle's causal forward, all within the 2e-2 bf16 gate."""
    from decoder_prefill_decode_amd import pipeline
    cfg = vs.scaled(vs.C3, n_layers=1, vocab=4101, seq=37, n_img=8, img_start=4, decode_steps=0, capacity=64,
                    name="c3_1layer_bf16_tails")
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, 0)]
    ref = od.run_decoder(cfg, glob, layers, steps=0)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.embed_inject()
    p0 = 0
    for s in (20, 3, 12, 2):
        run.model.prefill(run.x[p0:p0 + s], p0, run.cos, run.sin, [pipeline.causal_mask()], run.kv, run.ws)
        p0 += s
    assert p0 == cfg.seq and run.kv.len() == cfg.seq
    assert rel(run.x.cpu().numpy(), ref["prefill_x"]) <= 2e-2
    k, v = (t[:, :cfg.seq].float().cpu().numpy() for t in run.kv.kv(0))
    assert rel(k, ref["k_cache"][0][:, :cfg.seq]) <= 2e-2 and rel(v, ref["v_cache"][0][:, :cfg.seq]) <= 2e-2
    # head over rows 20..36 (17 rows: the row-tiled head) and over the last 12-row chunk (the few-row head)
    for r0 in (20, 23):
        rows = run.x[r0:r0 + (cfg.seq - r0 if r0 == 20 else 12)].contiguous()
        S = rows.shape[0]
        pred = torch.empty(S, dtype=torch.int32, device="cuda")
        logits = torch.empty((S, cfg.vocab), dtype=torch.float32, device="cuda")
        run.model.lmhead_argmax_rows(rows, pred, run.ws, logits)
        want = np.stack([od.lm_head_logits(ref["prefill_x"][r0 + i], glob["final_norm"], glob["embed"], cfg.eps, od.BF16)
                         for i in range(S)])
        assert rel(logits.cpu().numpy(), want) <= 2e-2
        assert [int(p) for p in pred.cpu()] == [int(np.argmax(r)) for r in logits.cpu().numpy()]


def test_graph_loop_continues_after_verify_commits():
    """fp32 4B-class layer shape (2 layers), a 160-slot window: verify commits interleaved with graph-loop
    decoding, the device length moving by several positions per commit and once across the 128 band
    boundary inside a verify block (prompt 100, verify 6 with a wrong draft at offset 2, 20 graph-loop steps,
    verify 8 all correct, 10 graph-loop steps): the 41 tokens are the oracle's greedy ids and the caches
    equal a one-token decode's (1e-4)."""
    from decoder_prefill_decode_amd import pipeline
    cfg = vs.scaled(vs.C4, n_layers=2, vocab=8192, seq=100, n_img=30, img_start=16, decode_steps=44, capacity=160,
                    dtype="f32", name="c4_2layer_f32_verify_loop")
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    ids = [int(i) for i in od.run_decoder(cfg, glob, layers)["ids"]]
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.prefill()
    gen = [int(run.first_token()[0])]

    def verify(k, wrong=()):
        i0 = len(gen) - 1
        draft = [gen[-1]] + ids[i0 + 1:i0 + k]
        for off in wrong:
            draft[off] = (draft[off] + 1) % (cfg.vocab - 1)
        toks, nxt = run.verify_block(draft)
        gen.extend(toks)
        run.tok.fill_(nxt)

    verify(6, wrong=(2,))
    assert run.kv.len() == cfg.seq + 2
    gen.extend(int(t) for t in run.decode(20, loop=True))
    verify(8)
    assert run.kv.len() == cfg.seq + 30 > 128
    gen.extend(int(t) for t in run.decode(10, loop=True))
    assert len(gen) == 41 and gen == ids[:41]
    ar = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    ar.prefill()
    ar.first_token()
    ar.decode(40, loop=False)
    T = run.kv.len()
    assert T == ar.kv.len() == cfg.seq + 40
    for l in range(cfg.n_layers):
        ka, va = (t[:, :T].cpu().numpy() for t in ar.kv.kv(l))
        kb, vb = (t[:, :T].cpu().numpy() for t in run.kv.kv(l))
        assert rel(kb, ka) <= 1e-4 and rel(vb, va) <= 1e-4
