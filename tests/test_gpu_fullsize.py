"""Full-size GPU parity against stored oracle results (tests/golden/*.npz,
written by tests/golden/make_golden.py, which calls only the oracle).

Decoder stacks (28-layer Qwen3-style and 36-layer 4B-class, bf16), element by
element against the exact-sum oracle, all at the bf16 gate 2e-2 (max relative
error over the tensor):
  * every prefill row and every first-token logit;
  * every valid K/V slot of layers 0, L/2 and L-1 after the prompt and after a
    decode teacher-forced on the oracle's ids (so decode slots are comparable);
  * greedy ids free-running and teacher-forced: exact at every step whose
    oracle top-2 margin is at least the oracle's own noise floor (the largest
    logit change of the oracle rerun with float32 sums, stored with the
    golden); the agreement counts are printed.
The 36-layer stack's deepest tensors (prefill rows after 36 layers, the
first-token logits, layer 35's K/V) are an expected failure of the 2e-2 gate:
the oracle's own float32-sum rerun already exceeds it there (C4_DEEP below).
Vision tower (27 layers + merger): every merged row, fp32 within 1e-4, the
bf16-storage tower (Mixed policy of the HunyuanOCR v1.5 port, §3.7) within 2e-2.
"""
import os

import numpy as np
import pytest
import torch

import vlm_synth as vs
from tests._parity import check_ids, rel

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BF16_GATE = 2e-2


def load(name):
    return dict(np.load(os.path.join(GOLDEN, f"{name}.npz"), allow_pickle=False))


def bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


# The 36-layer stack's deepest tensors sit at the edge of what its arithmetic fixes: the oracle rerun
# with float32 sums (operands and rounding points unchanged) already differs from the exact oracle by
# 2.29e-2 on the first-token logits and 2.03e-2 on layer 35's K/V (floors stored with the golden), above
# the 2e-2 gate. The gate is kept; the known exceedance of these tensors is an expected failure.
C4_DEEP = ("36-layer bf16 stack: the oracle's own float32-sum rerun moves the first-token logits by 2.29e-2 "
           "and layer 35's K/V by 2.03e-2 (above the 2e-2 gate), so no float32-accumulating implementation is "
           "bound to meet the gate on these tensors; the measured GPU figures are printed")
_RUNS = {}


def gpu_pass(cfg):
    """One GPU pass per stack: prefill, first token, free-running decode, then the cache truncated to
    the prompt and a decode teacher-forced on the oracle's ids (so decode slots are comparable)."""
    if cfg.name in _RUNS:
        return _RUNS[cfg.name]
    from decoder_prefill_decode_amd import pipeline
    g = load(cfg.name)
    glob = vs.decoder_globals(cfg)
    run = pipeline.DecoderRun(cfg, lambda l: vs.decoder_layer_weights(cfg, l), glob)
    x = run.prefill()
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    tok0 = int(run.first_token(logits)[0])
    r = {"g": g, "err_x": rel(x.cpu().numpy(), g["prefill_x"]), "err_lg": rel(logits.cpu().numpy(), g["logits0"])}
    r["free"] = [tok0] + [int(i) for i in run.decode(cfg.decode_steps)]
    run.kv.truncate(cfg.seq)
    r["forced"] = [tok0] + [int(i) for i in run.decode_forced(g["ids"][:-1])]
    T = cfg.seq + cfg.decode_steps
    k_ref, v_ref = bits_to_f32(g["k_bits"]), bits_to_f32(g["v_bits"])
    r["kv"] = {}
    for i, l in enumerate(g["kv_layers"]):
        k, v = run.kv.kv(int(l))
        k, v = k[:, :T].float().cpu().numpy(), v[:, :T].float().cpu().numpy()
        r["kv"][int(l)] = max(rel(k, k_ref[i]), rel(v, v_ref[i]))
    del run
    torch.cuda.empty_cache()
    print(f"{cfg.name}: prefill rows {r['err_x']:.3e} (oracle floor {float(g['floor_prefill_rel']):.3e}), "
          f"first-token logits {r['err_lg']:.3e}, KV per layer over all {T} slots "
          f"{ {l: round(e, 5) for l, e in r['kv'].items()} } (oracle floor "
          f"{[round(float(f), 5) for f in g['floor_kv_rel']]})")
    _RUNS[cfg.name] = r
    return r


@pytest.mark.parametrize("cfg", [vs.C3, vs.C4], ids=["c3_28layer", "c4_36layer"])
def test_decoder_stack_full_size_ids_and_cache(cfg):
    """Greedy ids (exact above the oracle's noise floor) and the K/V of layers 0 and L/2 at 2e-2."""
    r = gpu_pass(cfg)
    g = r["g"]
    check_ids(cfg.name, r["free"], r["forced"], g["ids"], g["margins"], float(g["floor_logit"]))
    shallow = {l: e for l, e in r["kv"].items() if l < cfg.n_layers - 1}
    assert all(e <= BF16_GATE for e in shallow.values()), shallow


@pytest.mark.parametrize("cfg", [vs.C3, pytest.param(vs.C4, marks=pytest.mark.xfail(reason=C4_DEEP, strict=False))],
                         ids=["c3_28layer", "c4_36layer"])
def test_decoder_stack_full_size_deep_tensors(cfg):
    """Every prefill row, every first-token logit and the last layer's K/V at the 2e-2 gate."""
    r = gpu_pass(cfg)
    last = r["kv"][cfg.n_layers - 1]
    assert r["err_x"] <= BF16_GATE and r["err_lg"] <= BF16_GATE and last <= BF16_GATE, \
        (r["err_x"], r["err_lg"], last)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_vit_full_size(dtype):
    from decoder_prefill_decode_amd import pipeline
    cfg = vs.C5 if dtype == "f32" else vs.scaled_vit(vs.C5, dtype=vs.BF16, name="c5_vit_27l_bf16")
    g = load(cfg.name)
    glob = vs.vit_globals(cfg)
    run = pipeline.VitRun(cfg, lambda l: vs.vit_layer_weights(cfg, l), glob)
    out = run.run().cpu().numpy()
    err = rel(out, g["out"])
    floor = f" (oracle floor {float(g['floor_out_rel']):.3e})" if "floor_out_rel" in g else ""
    print(f"{cfg.name}: merged-output max rel err {err:.3e}{floor}")
    assert err <= (1e-4 if dtype == "f32" else BF16_GATE), err
