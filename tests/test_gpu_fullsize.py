"""Full-size GPU parity against stored oracle results (tests/golden/*.npz,
written by tests/golden/make_golden.py, which calls only the oracle).

Decoder stacks (28-layer Qwen3-style and 36-layer 4B-class, bf16): sampled
prefill rows and the top-64 first-token logits within the bf16 gate (2e-2 of
the tensor's max); sampled KV slots within twice the oracle's own noise
floor at that depth; greedy ids checked free-running and teacher-forced, a
disagreement allowed only at a step whose oracle top-2 margin is below the
oracle's own first-token logit noise floor (see test_gpu_decoder.check_ids).
The noise floors (tests/golden/noise_floor.json, written by
tests/golden/noise_floor.py from the oracle alone) are the difference between
the oracle with float32 BLAS and with float64 products of the same bf16
operands: no result finer than that is fixed by the arithmetic.
Vision tower (27 layers + merger, fp32): sampled merged rows within 1e-4.
"""
import json
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


def noise_floor(name):
    with open(os.path.join(GOLDEN, "noise_floor.json")) as f:
        return json.load(f)[name]


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
    kv_err = []
    for i, l in enumerate(L):
        k, v = run.kv.kv(int(l))
        idx = torch.from_numpy(slots).to("cuda")
        ks, vv = k[:, idx].float().cpu().numpy(), v[:, idx].float().cpu().numpy()
        pr = slots < cfg.seq   # prompt slots; decode slots differ after a free-running divergence
        kv_err.append(max(np.abs(ks[:, pr] - g["k_samples"][i][:, pr]).max() / np.abs(g["k_samples"][i]).max(),
                          np.abs(vv[:, pr] - g["v_samples"][i][:, pr]).max() / np.abs(g["v_samples"][i]).max()))
    run.kv.truncate(cfg.seq)
    forced = [tok0] + list(run.decode_forced(g["ids"][:-1]))
    nf = noise_floor(cfg.name)
    eps = max(8 * float(err_lg), nf["logit_abs"])
    agree = sum(int(a == b) for a, b in zip(free, g["ids"]))
    print(f"{cfg.name}: prefill err {err_x:.2e}, top-logit err {err_lg:.2e}, KV err {kv_err}, tie eps {eps:.2e}, "
          f"free-running agreement {agree}/{len(free)}, "
          f"teacher-forced agreement {sum(int(a == b) for a, b in zip(forced, g['ids']))}/{len(forced)}")
    floor = [nf["kv_rel"][str(int(l))] for l in L]
    assert all(e <= 2 * f for e, f in zip(kv_err, floor)), (kv_err, floor)
    flips, div = check_ids(free, forced, g["ids"], g["margins"], eps)
    print(f"{cfg.name}: first divergence {div}, tie-ambiguous flips {flips}")


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
