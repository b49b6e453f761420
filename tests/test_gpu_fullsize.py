"""Full-size GPU parity against stored oracle results (tests/golden/*.npz,
written by tests/golden/make_golden.py, which calls only the oracle).

Decoder stacks (28-layer Qwen3-style and 36-layer 4B-class, bf16): sampled
prefill rows, the top-64 first-token logits and sampled KV slots within the
bf16 gate (2e-2 of the tensor's max), and greedy ids checked free-running and
teacher-forced with near-tie attribution (see test_gpu_decoder.check_ids).
Vision tower (27 layers + merger, fp32): sampled merged rows within 1e-4.
"""
import os

import numpy as np
import pytest
import torch

import vlm_synth as vs
from tests.test_gpu_decoder import check_ids

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    return dict(np.load(os.path.join(GOLDEN, f"{name}.npz"), allow_pickle=False))


@pytest.mark.parametrize("cfg", [vs.C3, vs.C4], ids=["c3_28layer", "c4_36layer"])
def test_decoder_stack_full_size(cfg):
    from decoder_prefill_decode_amd import pipeline
    g = load(cfg.name)
    glob = vs.decoder_globals(cfg)
    run = pipeline.DecoderRun(cfg, lambda l: vs.decoder_layer_weights(cfg, l), glob)
    x = run.prefill()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    tok0 = int(run.first_token(logits)[0])
    rows = g["prefill_rows"]
    xr = x[torch.from_numpy(rows).to("cuda")].cpu().numpy()
    err_x = np.abs(xr - g["prefill_x_rows"]).max() / g["prefill_x_absmax"]
    lg = logits.cpu().numpy()
    err_lg = np.abs(lg[g["logits0_top_idx"]] - g["logits0_top_val"]).max()
    assert err_x <= 2e-2, err_x
    assert err_lg / g["logits0_absmax"] <= 2e-2, err_lg
    free = [tok0] + list(run.decode(cfg.decode_steps))
    L, slots = g["kv_layers"], g["kv_slots"]
    for i, l in enumerate(L):
        k, v = run.kv.kv(int(l))
        ks = k[:, torch.from_numpy(slots).to("cuda")].float().cpu().numpy()
        vv = v[:, torch.from_numpy(slots).to("cuda")].float().cpu().numpy()
        # slots after a free-running divergence hold different tokens: compare the prompt part always
        pr = slots < cfg.seq
        assert np.abs(ks[:, pr] - g["k_samples"][i][:, pr]).max() / np.abs(g["k_samples"][i]).max() <= 2e-2
        assert np.abs(vv[:, pr] - g["v_samples"][i][:, pr]).max() / np.abs(g["v_samples"][i]).max() <= 2e-2
    run.kv.truncate(cfg.seq)
    forced = [tok0] + list(run.decode_forced(g["ids"][:-1]))
    eps = 8 * float(err_lg)
    flips, div = check_ids(free, forced, g["ids"], g["margins"], eps)
    agree = sum(int(a == b) for a, b in zip(free, g["ids"]))
    print(f"{cfg.name}: prefill err {err_x:.2e}, top-logit err {err_lg:.2e}, tie eps {eps:.2e}, "
          f"free-running agreement {agree}/{len(free)} (first divergence {div}), tie flips {flips}, "
          f"teacher-forced agreement {sum(int(a == b) for a, b in zip(forced, g['ids']))}/{len(forced)}")


def test_vit_full_size():
    from decoder_prefill_decode_amd import pipeline
    cfg = vs.C5
    g = load(cfg.name)
    glob = vs.vit_globals(cfg)
    run = pipeline.VitRun(cfg, lambda l: vs.vit_layer_weights(cfg, l), glob)
    out = run.run().cpu().numpy()
    units = g["units"]
    err = np.abs(out[units] - g["out_rows"]).max() / g["out_absmax"]
    assert err <= 1e-4, err
    assert np.allclose(np.linalg.norm(out, axis=1), g["out_row_norms"], rtol=1e-4)
    print(f"{cfg.name}: merged-output max rel err {err:.2e}")
