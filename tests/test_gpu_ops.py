"""GPU checks of individual steps and invariants through the C ABI."""
import ctypes as C

import numpy as np
import pytest
import torch

from oracle import decoder as od
from oracle import vit as ov
import vlm_synth as vs

pytestmark = pytest.mark.gpu


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.fixture(scope="module")
def mods():
    from decoder_prefill_decode_amd import native, pipeline, runtime
    return native, pipeline, runtime


def make(cfg):
    return vs.decoder_globals(cfg), [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]


# ---------------------------------------------------------------- RoPE tables
def test_rope_tables_match_oracle(mods):
    _, _, rt = mods
    rng = np.random.default_rng(0)
    cases = [(np.arange(2048)[None, :], np.zeros(64, np.int32), 1, 128, 1e6),
             (rng.integers(0, 92, size=(2, 300)), np.r_[np.zeros(18), np.ones(18)].astype(np.int32), 2, 72, 1e6),
             (rng.integers(0, 500, size=(4, 100)), np.repeat(np.arange(4), 16).astype(np.int32), 1, 128, 1.11588e7)]
    for pos, axes, seg, d, theta in cases:
        cos, sin = rt.rope_table(pos, axes, seg, d, theta)
        rc, rs = od.rope_tables(pos, axes, seg, d, theta)
        # the GPU rounds float64 angles' cos/sin to float: within one float ulp
        assert np.max(np.abs(cos.cpu().numpy() - rc)) <= 1.2e-7
        assert np.max(np.abs(sin.cpu().numpy() - rs)) <= 1.2e-7


# ---------------------------------------------------------------- masks
def test_additive_window_mask_equals_causal(mods):
    """The pages' finite additive mask (0 / -1e9) gives the causal result."""
    N, pipeline, rt = mods
    cfg = vs.scaled(vs.C2_F32, seq=200, decode_steps=0, capacity=256)
    glob, layers = make(cfg)
    a = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    xa = a.prefill().cpu().numpy()
    b = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    add = torch.from_numpy(od.window_mask(cfg.seq, 0, cfg.seq).astype(np.float32)).to("cuda")
    xb = b.prefill(mask=rt.additive_mask(add)).cpu().numpy()
    assert rel(xb, xa) <= 1e-6


def test_prefill_equals_decode_replay(mods):
    """Youtu-VL ncnn port, 结果展示: replaying the prompt through the decode path
    reproduces the parallel prefill (3.0e-7 relative there, CPU fp32)."""
    _, pipeline, _ = mods
    cfg = vs.scaled(vs.C2_F32, seq=160, decode_steps=0, capacity=256)
    glob, layers = make(cfg)
    a = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    xa = a.prefill().cpu().numpy()
    b = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    t0 = 100
    b.embed_inject()
    b.model.prefill(b.x[:t0], 0, b.cos, b.sin, [pipeline.causal_mask()], b.kv, b.ws)
    rows = b.x_in[t0:].contiguous()
    out = b.decode_hidden(rows).cpu().numpy()
    err = rel(out, xa[t0:])
    assert err <= 2e-6, err
    ka, va = a.kv.kv(0)
    kb, vb = b.kv.kv(0)
    assert rel(kb[:, :cfg.seq].cpu().numpy(), ka[:, :cfg.seq].cpu().numpy()) <= 2e-6


def test_chunked_prefill_equals_full(mods):
    """Prefill with pos0 > 0 over an existing cache (multi-token verify form)."""
    _, pipeline, _ = mods
    cfg = vs.scaled(vs.C3, n_layers=2, vocab=4096, seq=150, n_img=60, img_start=10, decode_steps=0, capacity=256)
    glob, layers = make(cfg)
    a = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    xa = a.prefill().cpu().numpy()
    b = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    b.embed_inject()
    for p0, s in ((0, 64), (64, 50), (114, 36)):
        b.model.prefill(b.x[p0:p0 + s], p0, b.cos, b.sin, [pipeline.causal_mask()], b.kv, b.ws)
    assert b.kv.len() == cfg.seq
    assert rel(b.x.cpu().numpy(), xa) <= 2e-2
    ref = od.run_decoder(cfg, glob, layers, steps=0)
    assert rel(b.x.cpu().numpy(), ref["prefill_x"]) <= 2e-2


# ---------------------------------------------------------------- lm_head edge cases
def _head_model(rt, V, H, dtype):
    m = rt.Model(n_layers=1, hidden=H, n_q_heads=2, n_kv_heads=1, head_dim=64, ffn=64, vocab=V, dtype=dtype)
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lmhead_argmax_ties_and_nonfinite(mods, dtype):
    _, _, rt = mods
    V, H = 5000, 256
    m = _head_model(rt, V, H, dtype)
    rng = np.random.default_rng(1)
    E = vs.to_bf16_values(rng.standard_normal((V, H)).astype(np.float32) * 0.02)
    E[1234] = E[4321] = E[77] * 0 + 0.5     # identical best rows: tie -> lowest index
    g = np.ones(H, np.float32)
    m.set_table(E, g)
    ws = m.workspace(1)
    x = torch.from_numpy(np.full(H, 0.3, np.float32)).to("cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(V, dtype=torch.float32, device="cuda")
    m.lmhead_argmax(x, tok, ws, logits)
    lg = logits.cpu().numpy()
    assert int(tok[0]) == int(np.argmax(lg)) == 1234
    ref = od.lm_head_logits(x.cpu().numpy(), g, E, 1e-6, od.BF16 if dtype == "bf16" else od.F64)
    assert rel(lg, ref) <= (2e-2 if dtype == "bf16" else 1e-4)
    xn = x.clone()
    xn[7] = float("nan")
    m.lmhead_argmax(xn, tok, ws)
    assert int(tok[0]) == -1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lmhead_argmax_rows_ties_pieces_and_nonfinite(mods, dtype):
    """The verify head's row argmax (partial keys over pieces of each row, then one reduction per
    row) on 5 rows of a 70001-entry table, so the last piece of every row is ragged:
    - row 0 ties the table rows 1234 and 60000, which lie in different pieces: the lowest index wins;
    - row 3's unique maximum is the table's last row;
    - row 2 holds a NaN, which gives -1.
    Every token equals numpy's first-maximum argmax of the logits the call returns."""
    _, _, rt = mods
    V, H, S = 70001, 256, 5
    m = _head_model(rt, V, H, dtype)
    rng = np.random.default_rng(4)
    E = vs.to_bf16_values(rng.standard_normal((V, H)).astype(np.float32) * 0.02)
    alt = np.where(np.arange(H) % 2 == 0, 1.0, -1.0).astype(np.float32)
    E[1234] = E[60000] = 0.5
    E[V - 1] = 0.5 * alt
    m.set_table(E, np.ones(H, np.float32))
    ws = m.workspace(S)
    xr = rng.standard_normal((S, H)).astype(np.float32)
    xr[0] = 0.3
    xr[3] = alt
    x = torch.from_numpy(xr).to("cuda")
    x[2, 11] = float("nan")
    tok = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    logits = torch.empty((S, V), dtype=torch.float32, device="cuda")
    m.lmhead_argmax_rows(x, tok, ws, logits)
    got = [int(t) for t in tok.cpu()]
    lg = logits.cpu().numpy()
    assert got[0] == 1234 and got[2] == -1 and got[3] == V - 1
    for r in (0, 1, 3, 4):
        assert got[r] == int(np.argmax(lg[r])), r
    tok2 = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    ws2 = torch.empty(ws.numel() + S * (H + V) * 4 + (1 << 16), dtype=torch.uint8, device="cuda")
    m.lmhead_argmax_rows(x, tok2, ws2)     # logits kept in the workspace: the same picks
    assert [int(t) for t in tok2.cpu()] == got


def test_lmhead_full_vocab_matches_oracle(mods):
    _, _, rt = mods
    cfg = vs.C3
    g = vs.decoder_globals(vs.scaled(cfg, seq=8, n_img=0))
    m = _head_model(rt, cfg.vocab, cfg.hidden, "bf16")
    m.set_table(g["embed"], g["final_norm"])
    ws = m.workspace(1)
    xr = np.random.default_rng(2).standard_normal(cfg.hidden).astype(np.float32)
    x = torch.from_numpy(xr).to("cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    m.lmhead_argmax(x, tok, ws, logits)
    lg = logits.cpu().numpy()
    ref = od.lm_head_logits(xr, g["final_norm"], g["embed"], cfg.eps, od.BF16)
    assert rel(lg, ref) <= 1e-5          # same bf16 operands, fp32 accumulation on both sides
    assert int(tok[0]) == int(np.argmax(lg)) == od.greedy_argmax(ref)


# ---------------------------------------------------------------- error paths leave the cache unchanged
def test_capacity_and_count_errors_leave_state(mods):
    N, pipeline, rt = mods
    cfg = vs.scaled(vs.C1, decode_steps=0, capacity=40)
    glob, layers = make(cfg)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.prefill()
    torch.cuda.synchronize()
    snap = run.kv.buf.clone()
    with pytest.raises(N.VlmError) as e:           # 32 + 16 rows > 40 slots
        run.model.prefill(run.x[:16], 32, run.cos, run.sin, [rt.causal_mask()], run.kv, run.ws)
    assert e.value.status == N.VLM_ERR_CAPACITY
    with pytest.raises(N.VlmError) as e:
        bad = glob["ids"].copy(); bad[0] = cfg.placeholder_id
        run.model.inject(run.x, bad, run.ids_dev, cfg.placeholder_id, run.img)
    assert e.value.status == N.VLM_ERR_COUNT_MISMATCH
    run.model.decode_loop(run.kv, run.cos, run.sin, run.ws, run.tok, 8, hist=run.hist)   # 32 + 8 = 40: fits
    with pytest.raises(N.VlmError) as e:
        run.model.decode_step(run.kv, run.cos, run.sin, run.ws, token_in=run.tok, token_out=run.tok)
    assert e.value.status == N.VLM_ERR_CAPACITY
    torch.cuda.synchronize()
    assert run.kv.len() == 40 and int(run.kv.device_len()[0]) == 40
    assert torch.equal(run.kv.buf[256:].view(torch.float32).view(2, 2, 2, 40, 64)[:, :, :, :32],
                       snap[256:].view(torch.float32).view(2, 2, 2, 40, 64)[:, :, :, :32])


def test_truncate_then_redecode_is_deterministic(mods):
    _, pipeline, _ = mods
    cfg = vs.C1
    glob, layers = make(cfg)
    run = pipeline.DecoderRun(cfg, lambda l: layers[l], glob)
    run.prefill()
    run.first_token()
    t0 = int(run.tok[0])
    a = run.decode(cfg.decode_steps)
    run.kv.truncate(cfg.seq)
    run.tok.fill_(t0)
    b = run.decode(cfg.decode_steps)
    assert list(a) == list(b)


# ---------------------------------------------------------------- vision tower
def test_vit_tower_and_merger_scaled_bf16(mods):
    """bf16 storage, fp32 accumulation (the Mixed policy of the HunyuanOCR v1.5 port, §3.7), with the
    72-wide heads zero-padded to the 16-wide MFMA steps inside the attention kernel."""
    _, pipeline, _ = mods
    cfg = vs.scaled_vit(vs.C5, n_layers=3, full_layers=(1,), dtype="bf16")
    glob = vs.vit_globals(cfg)
    layers = [vs.vit_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    ref = ov.run_vit(cfg, glob, layers)
    run = pipeline.VitRun(cfg, lambda l: layers[l], glob)
    out = run.run().cpu().numpy()
    ex, eo = rel(run.x.cpu().numpy(), ref["x_final"]), rel(out, ref["out"])
    print(f"bf16 tower: final rows {ex:.2e}, merged rows {eo:.2e}")
    assert ex <= 2e-2 and eo <= 2e-2


def test_vit_tower_and_merger_scaled(mods):
    _, pipeline, _ = mods
    cfg = vs.scaled_vit(vs.C5, n_layers=3, full_layers=(1,))
    glob = vs.vit_globals(cfg)
    layers = [vs.vit_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    ref = ov.run_vit(cfg, glob, layers)
    run = pipeline.VitRun(cfg, lambda l: layers[l], glob)
    out = run.run().cpu().numpy()
    assert rel(run.x.cpu().numpy(), ref["x_final"]) <= 1e-4
    assert rel(out, ref["out"]) <= 1e-4
