"""Non-finite results at the boundary (Penguin-VL ncnn port §4.1: a vocabulary /
logits mismatch there silently produced token 0; the library reports an
explicit VLM_ERR_NONFINITE instead).

A decode step whose argmax sees a NaN logit writes token -1, does not advance
the cache length and flags the cache header; vlm_kv_status reports it. The
valid cache slots and the length stay bit-identical, so decoding resumes from
the last good token exactly as if the failed step had never been issued.
"""
import numpy as np
import pytest
import torch

from oracle import decoder as od
import vlm_synth as vs

pytestmark = pytest.mark.gpu

CFG = vs.scaled(vs.C4, n_layers=2, vocab=8192, seq=80, n_img=30, img_start=16, decode_steps=6, capacity=128,
                dtype="f32", name="c4_2layer_f32_nan")


@pytest.fixture(scope="module")
def env():
    from decoder_prefill_decode_amd import native, pipeline
    glob = vs.decoder_globals(CFG)
    layers = [vs.decoder_layer_weights(CFG, l) for l in range(CFG.n_layers)]
    return native, pipeline, glob, layers


def snapshot(run, T):
    return [tuple(t[:, :T].clone() for t in run.kv.kv(l)) for l in range(CFG.n_layers)]


def same(a, b):
    return all(torch.equal(x, y) for pa, pb in zip(a, b) for x, y in zip(pa, pb))


def test_nan_decode_step_is_reported_and_not_committed(env):
    N, pipeline, glob, layers = env
    ref = od.run_decoder(CFG, glob, layers)
    run = pipeline.DecoderRun(CFG, lambda l: layers[l], glob)
    run.prefill()
    tok0 = int(run.first_token()[0])
    ids = [tok0] + [int(i) for i in run.decode(3, loop=False)]
    T = CFG.seq + 3
    before = snapshot(run, T)
    good_tok = run.tok.clone()
    nan_row = torch.full((CFG.hidden,), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    run.model.decode_step(run.kv, run.cos, run.sin, run.ws, x_in=nan_row, token_out=out)
    with pytest.raises(N.VlmError) as e:
        run.kv.status()
    assert e.value.status == N.VLM_ERR_NONFINITE and f"position {T}" in str(e.value)
    assert int(out[0]) == -1
    assert run.kv.len() == T and int(run.kv.device_len()[0]) == T
    assert same(before, snapshot(run, T))
    assert run.kv.status() == -1          # the flag was cleared by the report
    # decoding resumes from the last good token as if the failed step had not been issued
    run.tok.copy_(good_tok)
    ids += [int(i) for i in run.decode(CFG.decode_steps - 3, loop=True)]
    assert ids == [int(i) for i in ref["ids"]]


def test_invalid_token_in_graph_loop_fails_every_step(env):
    """Token -1 fed to the graph loop: its embedding row is NaN, so every step fails and none is
    committed; the status names the first position, the cache is unchanged."""
    N, pipeline, glob, layers = env
    run = pipeline.DecoderRun(CFG, lambda l: layers[l], glob)
    run.prefill()
    run.first_token()
    before = snapshot(run, CFG.seq)
    run.tok.fill_(-1)
    run.model.decode_loop(run.kv, run.cos, run.sin, run.ws, run.tok, 4, hist=run.hist)
    with pytest.raises(N.VlmError) as e:
        run.kv.status()
    assert e.value.status == N.VLM_ERR_NONFINITE and f"position {CFG.seq}" in str(e.value)
    assert run.kv.len() == CFG.seq and int(run.kv.device_len()[0]) == CFG.seq
    assert same(before, snapshot(run, CFG.seq))
    assert int(run.tok[0]) == -1


def test_nan_row_head_reports_nonfinite(env):
    N, pipeline, glob, layers = env
    run = pipeline.DecoderRun(CFG, lambda l: layers[l], glob)
    run.prefill()
    run.x[CFG.seq - 1, 7] = float("inf")
    with pytest.raises(N.VlmError) as e:
        run.first_token()
    assert e.value.status == N.VLM_ERR_NONFINITE and int(run.tok[0]) == -1
