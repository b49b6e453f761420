"""Writes noise_floor.json: how far the oracle moves when only its contraction
order changes (float32 BLAS vs float64 products of the same bf16 operands,
with every bf16 rounding point unchanged).

Calls only oracle/ and the shared input generators. The full-size GPU tests
use these numbers: a greedy step whose oracle top-2 margin is below the
logit floor is not decided by the arithmetic (two valid orderings of the
oracle itself can disagree), and KV-cache samples are gated at twice the
cache floor of their layer.

    python tests/golden/noise_floor.py c3_qwen3_28l c4_llama_4b
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import decoder as od  # noqa: E402
import vlm_synth as vs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noise_floor.json")


def lin_f64(a, w, prec):
    """The oracle's contraction with float64 products instead of float32 BLAS."""
    if prec == od.BF16:
        return od.bf16_round(a) @ w.astype(np.float64).T
    return np.asarray(a, np.float64) @ w.T


def floor(cfg):
    glob = vs.decoder_globals(cfg)
    layers = [vs.decoder_layer_weights(cfg, l) for l in range(cfg.n_layers)]
    a = od.run_decoder(cfg, glob, layers, steps=0)
    orig = od._lin
    od._lin = lin_f64
    try:
        b = od.run_decoder(cfg, glob, layers, steps=0)
    finally:
        od._lin = orig
    S = cfg.seq

    def rel(x, y):
        return float(np.abs(x - y).max() / np.abs(x).max())
    kv = {}
    for l in (0, cfg.n_layers - 1):
        kv[str(l)] = max(rel(a["k_cache"][l][:, :S], b["k_cache"][l][:, :S]),
                         rel(a["v_cache"][l][:, :S], b["v_cache"][l][:, :S]))
    return {"prefill_rel": rel(a["prefill_x"], b["prefill_x"]),
            "logit_abs": float(np.abs(a["logits0"] - b["logits0"]).max()),
            "logit_absmax": float(np.abs(a["logits0"]).max()), "kv_rel": kv}


if __name__ == "__main__":
    try:
        res = json.load(open(OUT))
    except (OSError, ValueError):
        res = {}
    for name in sys.argv[1:]:
        res[name] = floor(vs.ALL_CONFIGS[name])
        print(name, res[name], flush=True)
        with open(OUT, "w") as f:
            json.dump(res, f, indent=1)
